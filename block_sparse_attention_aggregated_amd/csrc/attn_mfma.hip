// Block-sparse (and dense) attention forward on gfx950 bf16 MFMA.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Forward-Only Sparse Execution" and "Complexity and Scope": each
// query block visits only the key blocks of its list, so the work scales with
// the retained fraction of blocks; softmax over the real keys of those blocks.
//
// Shape: bf16 Q/K/V, head_dim 128, query and key blocks of b = 64, 128 or 256
// tokens.  One workgroup of b / 32 wavefronts per query block (two workgroups
// per CU for b <= 128, one for b = 256); wavefront w owns queries 32w .. 32w+31
// of the block.  Each key block is processed as sub-tiles of 64 keys (32 at
// b = 64), double-buffered in LDS.  Per 64-key sub-tile:
//   S^T[key, query] = K Q^T   16 x v_mfma_f32_32x32x16_bf16 per wavefront in
//                             two independent accumulator chains (A = K from
//                             LDS, B = Q held in registers for the whole row),
//   online softmax in float32 registers: the MFMA output layout gives each
//     lane one query and 16 keys per 32-key tile; exp2 with sigma*log2(e)
//     folded into one FMA.  The softmax is optimistic: P is formed against the
//     current reference max without computing the sub-tile's own max; the
//     reference (the max of the first sub-tile) is only raised, with a rescale
//     of O and the sums, when a lane's P sum reaches 2^64 (row max: in-lane
//     max3 reduction plus one v_permlane32_swap with lane ^ 32).
//   P is rounded to bf16 once, and the row sum used to normalise O is taken
//     over those rounded values with v_dot2 (two per instruction), so the
//     weights the MFMA sees are normalised by their own sum; when the LSE is
//     asked for, the unrounded sum is kept beside it for that output,
//   O^T[d, query] += V^T P^T  16 MFMAs in four chains (A = V^T from LDS,
//                             B = P straight from the S^T register layout).
// Software pipeline, one step per sub-tile t, in two explicitly ordered phases:
//   phase 1: the S MFMAs of sub-tile t+1, each beside the exp2 / convert / sum
//            of two probabilities of sub-tile t;
//   phase 2: the P.V MFMAs of sub-tile t.
// LDS operand fragments are read two MFMAs ahead of their use.  K and V go
// from global memory straight into LDS with buffer_load_dwordx4 ... lds (no
// registers): the K of sub-tile t+2 and the V of sub-tile t+1 are fetched
// during step t, into four separately declared LDS buffers so that the
// compiler need not wait for them before reading the other buffers.
// V stays row-major in LDS; the V^T operand of the P.V MFMA is read with
// ds_read_b64_tr_b16, which hands lane j of each 16-lane group element j&3 of
// the 8-byte segments addressed by lanes (j>>2) + 4e: sixteen source lanes
// pointing at 4 keys x 16 features deliver 16 features x 4 keys.  Two such
// reads give a lane the eight keys 8*(r/4) + 4*half + r%4 that its P values
// (the S^T layout) hold.  K and V rows (256 B) have XOR-swizzled 16-byte
// chunks, chosen so that the MFMA operand reads of both are free of bank
// conflicts without padding.  One barrier per sub-tile.  The block lists are
// read through the scalar cache.
//
// XCD-aware row queues, run by a persistent grid.  Rows are queued per XCD: a
// head's query blocks are split into S contiguous segments of per = ceil(n_q / S)
// blocks; the queue of XCD x holds segment x % S of head
// (8 / S) j + x / S for j = 0, 1, ... in order, so the rows resident on one XCD
// are consecutive query blocks of one head, whose overlapping block lists share
// that XCD's L2, and the GPU works on 8 / S heads at a time, whose K and V stay
// in the Infinity Cache.  S = 4 at b = 128 and 256 with an even head count, 8
// otherwise (measured per block size).  Two ways to run the queues:
//   dynamic -- the grid holds as many workgroups as fit on the GPU at once (two
//              per CU at b = 128); each pops the next item of its own XCD's queue
//              (the XCC id register) with an atomic counter, runs that row, and
//              pops again; once its queue is empty it takes items from the other
//              queues, so uneven rows balance over the whole GPU and the launch
//              has no tail of one XCD's rows.  The per-workgroup set-up (lane
//              offsets, the zeroed V buffers) is done once, not once per row.
//              Needs kXcds counters in device memory, set at launch (each
//              workgroup's first row is item m of queue x for workgroup 8m + x,
//              taken without an atomic; the counters start past those).
//   static  -- one workgroup per item, without counters: workgroup 8m + x runs
//              item m of queue x, and the hardware dispatcher, which hands
//              consecutive workgroup ids to the XCDs round-robin and starts the
//              next one whenever a slot frees on that XCD, is the queue.  (A
//              persistent grid with a fixed share of rows per workgroup measured
//              slower than both: its workgroups drift apart, and the rows in
//              flight on an XCD stop being neighbours.)
// The dynamic queues run when the caller passes their counters and each XCD has
// at least two rounds of rows; otherwise the static ones.
// With a row order (uneven lists), each segment's rows run longest list first.

#include "sparstar_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace sparstar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int HD = 128;            // head_dim
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kBig = 18446744073709551616.0f;  // 2^64: bound on a lane's P sum per sub-tile
constexpr int kFragAhead = 2;      // MFMAs between an LDS operand read and its use

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}


// LDS: two K and two V sub-tile buffers, each [SUB keys][256 B] row-major.  They
// are four separate objects, and every LDS address below is derived from one of
// them, so the compiler can tell that a read of one buffer does not depend on
// the direct-to-LDS loads still in flight into another.
typedef __attribute__((address_space(3))) char lds_char;

typedef short v4s __attribute__((ext_vector_type(4)));

// s_waitcnt immediate (gfx9 encoding) that waits for lgkmcnt == 0 only:
// vmcnt = 63 (bits 3:0 and 15:14), expcnt = 7 (bits 6:4), lgkmcnt = 0 (bits 11:8).
constexpr int kWaitLgkm0 = 0xC07F;
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// Block size kB (queries and keys): kB / 32 wavefronts, sub-tiles of SUB keys.
// kB = 128: 4 wavefronts, 64-key sub-tiles (64 KB of LDS), two workgroups per CU;
// kB = 256: 8 wavefronts, one workgroup per CU; kB = 64: 2 wavefronts and 32-key
// sub-tiles (32 KB of LDS), four workgroups per CU.  Every case runs two
// wavefronts per SIMD (the second launch-bounds argument is waves per SIMD).
template <int kB>
struct Shape {
  static constexpr int BQ = kB, BK = kB;
  static constexpr int kWaves = kB / 32;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int SUB = kB == 64 ? 32 : 64;   // keys per LDS sub-tile
  static constexpr int kWavesPerSimd = 2;
  static constexpr int kSubs = kB / SUB;           // sub-tiles per key block
  static constexpr int kPasses = SUB / (4 * kWaves);  // load passes of 4 rows per wavefront per sub-tile
};

// The row queues of one launch (see the schedule above).
struct Sched {
  int per;         // query blocks per segment of a head
  int seg_shift;   // log2 of the segments per head
  int items;       // items per XCD queue: (heads / heads at a time, rounded up) * per
  int* ctr;        // dynamic queues: kXcds counters, set at launch; nullptr: static queues
};

struct Params {
  AttnArgs a;
  Sched sch;
};

// The kernel arguments, read through a pointer that the optimiser cannot follow:
// values taken from it are loaded where they are used (once per row), instead
// of being held in scalar registers for the whole persistent loop.
typedef const __attribute__((address_space(4))) Params* params_ptr;
__device__ inline params_ptr kernel_params() {
  params_ptr ap = (params_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ap));
  return ap;
}

template <int kB, bool kDense, bool kOutBf16, bool kLse>
__global__ __launch_bounds__(Shape<kB>::kThreads, Shape<kB>::kWavesPerSimd) void attn_mfma_kernel(Params prm) {
  constexpr int BQ = Shape<kB>::BQ, BK = Shape<kB>::BK;
  constexpr int kThreads = Shape<kB>::kThreads, kWaves = Shape<kB>::kWaves;
  constexpr int kPasses = Shape<kB>::kPasses;
  constexpr int SUB = Shape<kB>::SUB;
  constexpr int kTile = SUB * HD * 2;              // bytes per sub-tile buffer
  constexpr int NT = SUB / 32;                     // 32-key S tiles per sub-tile
  constexpr int N1 = 8 * NT;                       // S MFMAs (and softmax pairs) per sub-tile
  constexpr int N2 = SUB / 4;                      // P.V MFMAs per sub-tile
  __shared__ __attribute__((aligned(16))) char k_lds0[kTile];
  __shared__ __attribute__((aligned(16))) char k_lds1[kTile];
  __shared__ __attribute__((aligned(16))) char v_lds0[kTile];
  __shared__ __attribute__((aligned(16))) char v_lds1[kTile];
  __shared__ int s_item[3];                        // current item, its queue, queues found empty
  lds_char* const kb[2] = {(lds_char*)k_lds0, (lds_char*)k_lds1};
  lds_char* const vb[2] = {(lds_char*)v_lds0, (lds_char*)v_lds1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int l32 = lane & 31, hl = lane >> 5;
  const AttnArgs& a0 = prm.a;

  // ---- per-workgroup set-up, done once for all the rows the workgroup runs ----

  // K and V staging (direct to LDS): wavefront w, load pass t (0 .. kPasses - 1)
  // fills rows 4 kWaves t + 4w .. +4 of a sub-tile; lane i writes row + i/16 at
  // physical chunk i%16.  K rows hold logical chunk c at physical chunk
  // c ^ (row & 15); V rows at c ^ 4(row & 3), which moves whole 64-byte groups
  // (the 32-feature slices).
  const int st_row0 = 4 * wave + (lane >> 4);  // row in pass 0; pass t adds 4 kWaves t
  // In-head byte offsets fit in 32 bits (the host routes larger layouts elsewhere).
  const uint32_t ks_b = (uint32_t)a0.ks_t * 2u, vs_b = (uint32_t)a0.vs_t * 2u;  // bytes per key

  // LDS read offsets.  K: row kt*32 + l32, logical chunk 2ks + hl, physical chunk
  // (2ks + hl) ^ (row & 15) = 2ks ^ (hl ^ (l32 & 15)); kt adds 32 rows.
  const uint32_t k_row = l32 * (HD * 2), k_sw = hl ^ (l32 & 15);
  // The lane's offset for each feature step stays in a register for the whole
  // launch (the empty asm keeps the compiler from re-forming it with an add at
  // every read), so each K read is one ds_read_b128 with the buffer and the key
  // tile in its immediate offset.
  // The instances that also write the LSE hold two more sums per lane: they form
  // each offset at its read instead (from k_row and k_sw, which the step re-takes
  // through an empty asm so that the offsets are not hoisted), which keeps them
  // within 256 VGPRs without spilling to scratch.
  uint32_t kr_off[HD / 16];
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) {
    kr_off[ks] = k_row + (((2 * ks) ^ k_sw) << 4);
    if (!kLse) asm volatile("" : "+v"(kr_off[ks]));
  }
  uint32_t k_row_l = k_row, k_sw_l = k_sw;
  // V^T operand by transposing reads.  Lane L = 16g + m points at key
  // 16ks + 8r + 4(g >> 1) + (m >> 2) (r = 0, 1 for the two reads of a step) and
  // features 32dt + 16(g & 1) + 4(m & 3) .. +4: chunk 4dt + cc, cc = 2(g & 1) + (m & 3) / 2,
  // byte 8 (m & 1) in it; physical chunk (4dt + cc) ^ 4(kr & 3) with kr = 4(g >> 1) + (m >> 2)
  // (keys 16ks + 8r + kr share row & 3), i.e. (cc ^ 4(kr & 3)) ^ 4dt.  The 32 lanes
  // one LDS cycle serves (g = 0, 1, or 2, 3) read 4 keys x 32 features, whose four
  // 64-byte groups land in the four distinct group slots of the 256-byte bank
  // window: no bank conflicts.
  uint32_t v_tr[HD / 32];
  {
    const int g16 = lane >> 4, m16 = lane & 15;
    const int kr = 4 * (g16 >> 1) + (m16 >> 2);
    const int cx = (2 * (g16 & 1) + ((m16 & 3) >> 1)) ^ (4 * (kr & 3));
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
      v_tr[dt] = (uint32_t)(kr * (HD * 2) + ((cx ^ (4 * dt)) << 4) + 8 * (m16 & 1));
  }
  uint32_t k_off[kPasses], v_off[kPasses];  // per load pass: row offset + swizzled chunk
  #pragma unroll
  for (int t = 0; t < kPasses; ++t) {
    const int row = st_row0 + 4 * kWaves * t;
    k_off[t] = (uint32_t)row * ks_b + (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
    v_off[t] = (uint32_t)row * vs_b + (uint32_t)(((lane & 15) ^ (4 * (row & 3))) * 16);
  }
  // The V buffers start as zeros, so the rows past the end of a partial tile
  // (which the loads leave alone) always hold finite values: zeros or an earlier
  // tile's values, of this row or an earlier one.
  {
    typedef int v4i __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i* lds_v4i;
  #pragma unroll
    for (int i = 0; i < kTile / 16 / kThreads; ++i) {
      *(lds_v4i)(vb[0] + (i * kThreads + tid) * 16) = v4i{0, 0, 0, 0};
      *(lds_v4i)(vb[1] + (i * kThreads + tid) * 16) = v4i{0, 0, 0, 0};
    }
  }

  // ---- the row queue ----
  // An item m of queue x is query block mm = m % per of segment x % S of head
  // (8 / S)(m / per) + x / S, S = 1 << seg_shift; with a row order, the segment's
  // mm-th longest row instead.
  // The current item and its queue live in LDS, written by thread 0 and read by
  // every thread after a barrier, so that nothing of the queue stays in registers
  // while a row runs.
  auto next_item = [&](bool first) {
    // The first barrier keeps thread 0 from overwriting an item not yet read by all.
    __syncthreads();
    if (tid == 0) {
      const auto& sch = kernel_params()->sch;
      int q, m;
      if (sch.ctr != nullptr && first) {
        // Dynamic, first row: workgroup 8m + x takes item m of queue x without an
        // atomic (the counters start at the W = gridDim / 8 items taken this way),
        // so the launch does not open with W atomics queued on each counter.
        q = (int)(blockIdx.x & (kXcds - 1));
        m = (int)(blockIdx.x / kXcds);
        s_item[2] = 0;
      } else if (sch.ctr != nullptr) {
        // Dynamic: one atomic pop on the queue of the XCD the workgroup runs on (the
        // XCC id register); an empty queue sends it on to the next XCD's.  s_item[2]
        // counts the queues found empty so far.
        q = s_item[2] == 0 ? (__builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcds - 1))  // hwreg(HW_REG_XCC_ID, 0, 4)
                           : s_item[1];
        int tries = s_item[2];
        m = -1;
        while (tries < kXcds) {
          m = atomicAdd(sch.ctr + q, 1);
          if (m < sch.items) break;
          m = -1;
          q = (q + 1) & (kXcds - 1);
          ++tries;
        }
        s_item[2] = tries;
      } else {
        // Static: workgroup 8m + x runs item m of queue x (one item per workgroup).
        q = (int)(blockIdx.x & (kXcds - 1));
        m = first ? (int)(blockIdx.x / kXcds) : s_item[0] + (int)(gridDim.x / kXcds);
      }
      s_item[0] = m;
      s_item[1] = q;
    }
    __syncthreads();
  };

  next_item(true);
#pragma unroll 1
  for (;; next_item(false)) {
    const int item = __builtin_amdgcn_readfirstlane(*(volatile int*)&s_item[0]);
    const int queue = __builtin_amdgcn_readfirstlane(*(volatile int*)&s_item[1]);
    if (item < 0 || item >= kernel_params()->sch.items) break;
    // Dynamic queues: keep the rows in flight on an XCD in step.  The SIMD
    // arbiter favours the older wavefront, and a persistent workgroup never gets
    // younger, so without a correction some workgroups fall steadily behind (the
    // start times of the W rows resident on an XCD spread by about 6 us per row
    // they run, to ~200 us at 720p), neighbouring rows stop reading the same key
    // blocks at the same time, and the L2 hit rate of the K/V tiles drops from
    // 75% to 71.5%.  The items of an XCD are popped in finishing order, so a row
    // popped in the later half of its round (item mod W >= W/2, W workgroups per
    // XCD) belongs to a workgroup that is behind: it runs at raised wave
    // priority, which bounds the spread (~50 us) and restores the hit rate.
    if (kernel_params()->sch.ctr != nullptr) {
      const int w = (int)(gridDim.x / kXcds);
      if (item % w >= w / 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    const auto& a = kernel_params()->a;
    const auto& sch = kernel_params()->sch;
    const float c = a.sigma * kLog2e;
    const auto& g = a.g;
    const int hset = item / sch.per, mm = item - hset * sch.per;
    const int64_t bh = ((int64_t)hset << (3 - sch.seg_shift)) + (queue >> sch.seg_shift);
    if (bh >= (int64_t)g.B * g.H) continue;  // uniform over the workgroup
    const int seg = queue & ((1 << sch.seg_shift) - 1);
    const int qi = a.row_order ? a.row_order[((bh << sch.seg_shift) + seg) * sch.per + mm] : seg * sch.per + mm;
    if (qi < 0 || qi >= g.n_q) continue;  // uniform over the workgroup
    const int64_t row = bh * g.n_q + qi;
    const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);

    const __bf16* qbase = static_cast<const __bf16*>(a.q) + bi * a.qs_b + hi * a.qs_h;
    const char* kbase = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.k) + bi * a.ks_b + hi * a.ks_h);
    const char* vbase = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.v) + bi * a.vs_b + hi * a.vs_h);

    // Q^T operand: lane holds query l32 of this wavefront, features 16*ks + 8*hl .. +8.
    const int64_t qrow = (int64_t)qi * BQ + wave * 32 + l32;
    const bool q_valid = qrow < g.L_q;
    bf16x8 qf[HD / 16];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
      const uint4 raw = q_valid ? ld16(qbase + qrow * a.qs_t + ks * 16 + hl * 8) : make_uint4(0, 0, 0, 0);
      qf[ks] = as_bf16x8(raw);
    }

    f32x16 o[HD / 32];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    // l: sum of the bf16-rounded P (normalises O); l_exact: unrounded sum (for the LSE).
    float m_run = -INFINITY, l = 0.f, l_exact = 0.f;

    // The block lists are read-only here: read them through the scalar cache.
    typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
    const cint_ptr rp = (cint_ptr)a.row_ptr;
    cint_ptr ci = (cint_ptr)a.col_idx;
    // The values the list walk needs, taken once per row; the empty asm makes them
    // plain register values, which the compiler keeps instead of reloading them
    // from the kernel arguments inside the walk.
    int L_k = (int)g.L_k, n_k = g.n_k;
    asm volatile("" : "+s"(L_k), "+s"(n_k), "+s"(ci));
    // List positions fit in 32 bits: row_ptr entries are int32.
    int beg = 0, end = n_k;
    if (!kDense) {
      beg = rp[row];
      end = rp[row + 1];
      if (beg < 0) beg = 0;
      if ((int64_t)end > a.col_idx_len) end = (int)a.col_idx_len;
    }
    // A sub-tile: the SUB keys from token tok on, of the key block at list position p
    // (p >= end: past the end of the list).  tok is a multiple of SUB; its key block
    // is tok / BK.
    struct Sub {
      int p, tok, jn;  // jn: the list entry at p + 1, read ahead (or -1)
    };
    // Real keys of a sub-tile: 1 .. SUB, or 0 past the end of the list.
    auto sub_len = [&](const Sub& s) -> int { return s.p < end ? min(SUB, L_k - s.tok) : 0; };
    // First sub-tile of the first in-range list entry at or after p; each entry is
    // read once.
    auto first_sub = [&](int p) -> Sub {
      int j = (int)p;
      if (!kDense) {
        j = 0;
        while (p < end) {
          j = ci[p];
          if (j >= 0 && j < n_k) break;
          ++p;
        }
      }
      return Sub{p, p < end ? j * BK : 0, -1};
    };
    // The sub-tile after s: the next one of the same key block while that block has
    // real keys left, else the first of the next in-range list entry.  The step that
    // enters a block's last sub-tile reads the next list entry, so the step that
    // leaves the block finds it in a register.
    auto advance = [&](const Sub& s) -> Sub {
      if (s.p >= end) return s;
      const int in_blk = s.tok & (BK - 1);
      if (in_blk + SUB < BK && L_k - s.tok > SUB) {
        if (kDense || in_blk + 2 * SUB < BK) return Sub{s.p, s.tok + SUB, s.jn};
        return Sub{s.p, s.tok + SUB, s.p + 1 < end ? ci[s.p + 1] : -1};
      }
      if (!kDense && s.jn >= 0 && s.jn < n_k) return Sub{s.p + 1, s.jn * BK, -1};
      return first_sub(s.p + 1);
    };

    // K and V go straight to LDS through buffer resources, one per sub-tile: base =
    // its first row, range = its real rows.  Lanes of rows past the end of a
    // partial sub-tile fall outside the range and read zeros, and so do all lanes
    // of the sub-tiles past the end of the list (range 0; their buffers are not
    // read).  Every tile is then the same four loads, with no branch and no
    // per-lane select, which also lets the compiler track exactly which LDS
    // buffer each load writes (a direct-to-LDS global load would turn every LDS
    // wait issued while it is in flight into lgkmcnt(0)).  Scores of rows past
    // the end are masked to -inf, so their probabilities are exactly 0; V rows
    // there hold zeros or an earlier tile's finite values.
    auto load_tile = [&](const char* base, uint32_t stride_b, const uint32_t* off, const Sub& s,
                         lds_char* buf) {
      const char* first = base + (size_t)((uint32_t)s.tok * stride_b);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(first), (short)0, (int)((uint32_t)sub_len(s) * stride_b), kBufferFlags);
      // The per-wavefront LDS offset is hidden from the optimiser here so that the
      // M0 values are formed in the loop by one scalar add each, rather than hoisted
      // out of it (where they would be spilled to vector-register lanes).
      uint32_t woff = 4u * wave * (HD * 2);
      asm volatile("" : "+s"(woff));
      lds_char* const ldsb = buf + woff;
    #pragma unroll
      for (int t = 0; t < kPasses; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, ldsb + t * 4 * kWaves * (HD * 2), 16, off[t], 0, 0, 0);
    };
    auto load_k = [&](const Sub& s, lds_char* buf) { load_tile(kbase, ks_b, k_off, s, buf); };
    auto load_v = [&](const Sub& s, lds_char* buf) { load_tile(vbase, vs_b, v_off, s, buf); };
    auto k_frag = [&](lds_char* buf, int kt, int ks) -> bf16x8 {
      typedef const __attribute__((address_space(3))) bf16x8* lds_bf16x8;
      if (kLse) return *(lds_bf16x8)(buf + kt * 32 * (HD * 2) + k_row_l + (((2 * ks) ^ k_sw_l) << 4));
      return *(lds_bf16x8)(buf + kt * 32 * (HD * 2) + kr_off[ks]);
    };
    auto v_frag = [&](lds_char* buf, int dt, int ks) -> bf16x8 {
      typedef __attribute__((address_space(3))) v4s* lds_v4s;
      lds_char* const base = buf + ks * 16 * (HD * 2) + v_tr[dt];
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(base));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(base + 8 * (HD * 2)));
      bf16x8 r;
      __builtin_memcpy(&r, &lo, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
      return r;
    };
    // S^T of one sub-tile from K buffer buf (two 32-key tiles, eight 16-feature
    // steps); used once per row, before the pipelined loop.
    auto compute_s = [&](lds_char* buf, f32x16 (&s)[SUB / 32]) {
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks)
#pragma unroll
        for (int kt = 0; kt < SUB / 32; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(buf, kt, ks), qf[ks], ks == 0 ? f32x16{} : s[kt],
                                                          0, 0, 0);
    };
    // Scores of keys past the end of a partial sub-tile become -inf.  Register r of
    // tile kt holds key kt*32 + 8(r/4) + 4hl + r%4; the lane part moves into the limit
    // so that the per-register part stays an immediate.
    auto mask_tail = [&](f32x16 (&s)[SUB / 32], int len) {
      const int lim = len - 4 * hl;
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[kt][r] = -INFINITY;
    };
    // Max over the two lanes that hold one query (lane and lane ^ 32).
    auto pair_max = [](float x) -> float {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto tile_max = [&](const f32x16 (&s)[SUB / 32]) -> float {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kt][r]), s[kt][r + 1]);
      return pair_max(mx);
    };

    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // S of the current and the next sub-tile; the two arrays swap roles every step.
    f32x16 sA[SUB / 32], sB[SUB / 32];

    // Prologue: sub-tiles c0 (K and V), c1 (K) in flight; S of c0.  The reference
    // max starts at the max of c0.  The LDS buffers are free: the last step of
    // the previous row (or the set-up) ended with a barrier.
    Sub cur = first_sub(beg);
    Sub nxt = advance(cur);
    if (cur.p < end) {
      load_k(cur, kb[0]);
      load_v(cur, vb[0]);
      load_k(nxt, kb[1]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (cur.p < end) {
      compute_s(kb[0], sA);
      const int len0 = sub_len(cur);
      if (len0 < SUB) mask_tail(sA, len0);
      m_run = tile_max(sA);
    }
    __syncthreads();

    // Probabilities of one sub-tile against the reference max (mc = m_run * c):
    // pair i of the P operands from scores 2i, 2i + 1, plus the row sums.
    union PTile {
      bf16x8 v[SUB / 16];
      bf16x2 q[SUB / 4];
    };
    auto p_pair = [&](const f32x16 (&s)[SUB / 32], int i, float mc, PTile& pu, float& rs0, float& rs1, float& le) {
      const int t = i >> 3, r = 2 * (i & 7);
      f32x2 f;
      f[0] = __builtin_amdgcn_exp2f(fmaf(s[t][r], c, -mc));
      f[1] = __builtin_amdgcn_exp2f(fmaf(s[t][r + 1], c, -mc));
      if (kLse) le += f[0] + f[1];
      pu.q[i] = __builtin_convertvector(f, bf16x2);
      if (t == 0) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pu.q[i], ones, rs0, false);
      else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pu.q[i], ones, rs1, false);
    };

    // One pipeline step for the sub-tile with sequence parity PAR.  On entry: its
    // S is in registers, its V is in V buffer PAR and the next sub-tile's K in K
    // buffer PAR ^ 1.  The step fetches the K of the sub-tile after next into K
    // buffer PAR and the next V into V buffer PAR ^ 1, then runs two explicitly
    // ordered phases (sched_barrier keeps the order):
    //   phase 1: 16 MFMAs of S(next), each beside the softmax of two P values of
    //            this sub-tile; K fragments are read two MFMAs ahead;
    //   phase 2: 16 MFMAs of O += V^T P^T; V fragments are read two MFMAs ahead.
    // The softmax is optimistic: P is computed against the current reference max
    // without looking at this sub-tile's max.  Only if a lane's sum of the new P
    // reaches 2^64 (so some P may be large, or infinite) is the sub-tile redone:
    // its max (over both lanes of the query) becomes the reference, O and the sums
    // are rescaled, and P is recomputed.  Below that bound every P < 2^64, and O
    // and the sums (at most 2^17 keys) stay far inside the float32 range; the
    // normalisation by the sum at the end is unchanged by the choice of reference.
    auto step = [&](auto par) {
      constexpr int PAR = decltype(par)::value;
      lds_char* const k_cur = kb[PAR];
      lds_char* const k_nxt = kb[PAR ^ 1];
      lds_char* const v_cur = vb[PAR];
      lds_char* const v_nxt = vb[PAR ^ 1];
      f32x16(&s_cur)[SUB / 32] = PAR == 0 ? sA : sB;
      f32x16(&s_nxt)[SUB / 32] = PAR == 0 ? sB : sA;
      if (kLse) asm volatile("" : "+v"(k_row_l), "+v"(k_sw_l));
      const Sub nn = advance(nxt);
      load_k(nn, k_cur);
      load_v(nxt, v_nxt);
      const float mc = m_run * c;

      // Phase 1.  MFMA i: key tile i & 1, feature step i >> 1.  P values 2i, 2i + 1
      // (tile i >> 3, registers 2(i & 7), +1) form pair i & 3 of P operand i >> 2.
      // Drain the scalar loads of the block list first: their returns are unordered,
      // and with none pending every LDS wait below counts only the LDS reads ahead
      // of it (lgkmcnt(n) rather than lgkmcnt(0)).  vmcnt and expcnt: no wait.
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      constexpr int AH = kFragAhead, RING = kFragAhead + 1;
      bf16x8 kf[RING], vf[RING];
#pragma unroll
      for (int j = 0; j < AH; ++j) kf[j] = k_frag(k_nxt, j % NT, j / NT);
      PTile pu;
      float rs0 = 0.f, rs1 = 0.f, le_t = 0.f;
      // The softmax of pair i runs in three stages over three iterations (FMA in
      // i - 2, exp2 in i - 1, convert and sum in i), so no instruction waits on the
      // one issued just before it.
      auto st_a = [&](int i) -> f32x2 {
        const int t = i >> 3, r = 2 * (i & 7);
        f32x2 x;
        x[0] = fmaf(s_cur[t][r], c, -mc);
        x[1] = fmaf(s_cur[t][r + 1], c, -mc);
        return x;
      };
      auto st_b = [&](f32x2 x) -> f32x2 {
        f32x2 e;
        e[0] = __builtin_amdgcn_exp2f(x[0]);
        e[1] = __builtin_amdgcn_exp2f(x[1]);
        return e;
      };
      f32x2 x_1 = st_a(1), e_0 = st_b(st_a(0));
#pragma unroll
      for (int i = 0; i < N1; ++i) {
        if (i + AH < N1) kf[(i + AH) % RING] = k_frag(k_nxt, (i + AH) % NT, (i + AH) / NT);
        else vf[i + AH - N1] = v_frag(v_cur, (i + AH - N1) & 3, (i + AH - N1) >> 2);
        const int kt = i % NT, ks = i / NT;
        s_nxt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % RING], qf[ks], ks == 0 ? f32x16{} : s_nxt[kt], 0,
                                                            0, 0);
        const f32x2 x_2 = i + 2 < N1 ? st_a(i + 2) : f32x2{};
        const f32x2 e_1 = i + 1 < N1 ? st_b(x_1) : f32x2{};
        if (kLse) le_t += e_0[0] + e_0[1];
        pu.q[i] = __builtin_convertvector(e_0, bf16x2);
        if (i < 8) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pu.q[i], ones, rs0, false);
        else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pu.q[i], ones, rs1, false);
        e_0 = e_1;
        x_1 = x_2;
        __builtin_amdgcn_sched_barrier(0);
      }
      // Keep the softmax above in phase 1: without this, the compiler sinks it past
      // the branches below, next to its first use.
      if constexpr (NT == 2)
        asm volatile("" : "+v"(pu.v[0]), "+v"(pu.v[1]), "+v"(pu.v[2]), "+v"(pu.v[3]), "+v"(rs0), "+v"(rs1));
      else
        asm volatile("" : "+v"(pu.v[0]), "+v"(pu.v[1]), "+v"(rs0), "+v"(rs1));
      if (__any(rs0 + rs1 >= kBig)) {
        const float m_new = fmaxf(m_run, tile_max(s_cur));
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        l *= alpha;
        if (kLse) l_exact *= alpha;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m_run = m_new;
        rs0 = rs1 = le_t = 0.f;
#pragma unroll
        for (int i = 0; i < N1; ++i) p_pair(s_cur, i, m_run * c, pu, rs0, rs1, le_t);
      }
      l += rs0 + rs1;
      if (kLse) l_exact += le_t;
      const int len_nxt = sub_len(nxt);
      if (len_nxt < SUB) mask_tail(s_nxt, len_nxt);

      // Phase 2.  MFMA i: feature tile i & 3, key step i >> 2.
#pragma unroll
      for (int i = 0; i < N2; ++i) {
        if (i + AH < N2) vf[(i + AH) % RING] = v_frag(v_cur, (i + AH) & 3, (i + AH) >> 2);
        const int dt = i & 3, ks = i >> 2;
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % RING], pu.v[ks], o[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      __builtin_amdgcn_s_waitcnt(0);  // the K and V of later sub-tiles have landed in LDS
      __syncthreads();
      cur = nxt;
      nxt = nn;
    };

#pragma unroll 1
    while (cur.p < end) {
      step(std::integral_constant<int, 0>());
      if (cur.p >= end) break;
      step(std::integral_constant<int, 1>());
    }

    // Epilogue: the two lanes of a query hold partial row sums of disjoint keys.  The
    // output pointer, strides and scale are read again from the kernel arguments
    // (the empty asm hides where the pointer came from), so that they need not stay
    // in scalar registers through the loop.
    const auto* ap = &kernel_params()->a;
    const int bo = (int)(bh / ap->g.H), ho = (int)(bh - (int64_t)bo * ap->g.H);
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float le = kLse ? l_exact + __shfl_xor(l_exact, 32) : 0.f;
    if (q_valid) {
      if (kOutBf16) {
        __bf16* orow = static_cast<__bf16*>(ap->out) + bo * ap->os_b + ho * ap->os_h + qrow * ap->os_t;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[dt][gq * 4 + e] * inv);
            *reinterpret_cast<bf16x4*>(orow + dt * 32 + gq * 8 + hl * 4) = v4;
          }
      } else {
        float* orow = static_cast<float*>(ap->out) + bo * ap->os_b + ho * ap->os_h + qrow * ap->os_t;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float4 v4 = make_float4(o[dt][gq * 4] * inv, o[dt][gq * 4 + 1] * inv, o[dt][gq * 4 + 2] * inv,
                                    o[dt][gq * 4 + 3] * inv);
            *reinterpret_cast<float4*>(orow + dt * 32 + gq * 8 + hl * 4) = v4;
          }
      }
      if (kLse && hl == 0) ap->lse[bh * ap->g.L_q + qrow] = le > 0.f ? m_run * ap->sigma + __logf(le) : -INFINITY;
    }
  }
}

// Workgroups per XCD that fit at once on the current device: CUs per XCD times
// workgroups per CU (kept per device once known; 0 on failure).
template <int kB, bool kDense, bool kOutBf16, bool kLse>
int resident_per_xcd() {
  constexpr int kDevices = 64;
  static std::atomic<int> known[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 0;
  const int v = known[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_kernel<kB, kDense, kOutBf16, kLse>,
                                                   Shape<kB>::kThreads, 0) != hipSuccess)
    return 0;
  const int r = (cus / kXcds) * per_cu;
  if (r > 0) known[dev].store(r, std::memory_order_relaxed);
  return r;
}

// Queue counters at launch: the first `taken` items of every queue are the
// workgroups' first rows, handed out without atomics.
__global__ void init_counters_kernel(int* ctr, int n, int taken) {
  if ((int)threadIdx.x < n) ctr[threadIdx.x] = taken;
}

template <int kB, bool kDense, bool kOutBf16, bool kLse>
hipError_t launch(const AttnArgs& a, int* counters, hipStream_t s) {
  const int64_t bh_count = (int64_t)a.g.B * a.g.H;
  const int seg_count = segments_per_head(kB, bh_count);
  const int heads_at_once = kXcds / seg_count;
  Sched sch;
  sch.per = (a.g.n_q + seg_count - 1) / seg_count;
  sch.seg_shift = __builtin_ctz((unsigned)seg_count);  // seg_count is a power of two
  const int64_t items = (bh_count + heads_at_once - 1) / heads_at_once * sch.per;
  if (items > 0x7fffffffll) return hipErrorInvalidValue;
  sch.items = (int)items;
  // Dynamic queues: as many workgroups as fit at once.  Static: one workgroup per
  // item, so the hardware dispatcher, which starts workgroup 8m + x on XCD x as
  // soon as a slot there frees, runs each XCD's items in order.
  // The queues pay only with at least two rounds of rows per XCD: with fewer, the
  // grid is the rows themselves either way, and idle workgroups would only probe
  // the other XCDs' counters (measured 16% slower on a 0.2 ms scale of 640 rows).
  int64_t grid = (int64_t)kXcds * items;
  if (counters) {
    const int per_xcd = resident_per_xcd<kB, kDense, kOutBf16, kLse>();
    if (per_xcd <= 0) return hipErrorInvalidDeviceFunction;
    if (items >= 2 * (int64_t)per_xcd)
      grid = (int64_t)kXcds * per_xcd;
    else
      counters = nullptr;
  }
  if (grid > 0xffffffffll) return hipErrorInvalidValue;
  sch.ctr = counters;
  if (counters)
    hipLaunchKernelGGL(init_counters_kernel, dim3(1), dim3(64), 0, s, counters, kXcds, (int)(grid / kXcds));
  Params prm;
  prm.a = a;
  prm.sch = sch;
  hipLaunchKernelGGL((attn_mfma_kernel<kB, kDense, kOutBf16, kLse>), dim3((unsigned)grid),
                     dim3(Shape<kB>::kThreads), 0, s, prm);
  return hipSuccess;
}

template <int kB, bool kDense, bool kOutBf16>
hipError_t launch2(const AttnArgs& a, int* ctr, hipStream_t s) {
  return a.lse ? launch<kB, kDense, kOutBf16, true>(a, ctr, s) : launch<kB, kDense, kOutBf16, false>(a, ctr, s);
}

template <int kB>
hipError_t launch_b(const AttnArgs& a, int* ctr, hipStream_t s) {
  const bool dense = a.row_ptr == nullptr;
  const bool ob = a.out_dtype == 0;
  return dense ? (ob ? launch2<kB, true, true>(a, ctr, s) : launch2<kB, true, false>(a, ctr, s))
               : (ob ? launch2<kB, false, true>(a, ctr, s) : launch2<kB, false, false>(a, ctr, s));
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, int* counters, hipStream_t s) {
  if (a.g.D != HD || a.dtype != 0) return hipErrorInvalidValue;
  hipError_t e;
  switch (a.g.b) {
    case 64: e = launch_b<64>(a, counters, s); break;
    case 128: e = launch_b<128>(a, counters, s); break;
    case 256: e = launch_b<256>(a, counters, s); break;
    default: return hipErrorInvalidValue;
  }
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace sparstar
