// K3/K4: block-sparse (and dense) attention forward on gfx950 bf16 MFMA.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Forward-Only Sparse Execution" and "Complexity and Scope": each
// query block visits only the key blocks of its list, so the work scales with
// the retained fraction of blocks; softmax over the real keys of those blocks.
//
// Shape: bf16 Q/K/V, head_dim 128, 128-token query and key blocks.
// One workgroup (4 wavefronts) per query block, two workgroups per CU;
// wavefront w owns queries 32w .. 32w+31 of the block.  Each 128-key block
// is processed as two 64-key sub-tiles, double-buffered in LDS.  Per sub-tile:
//   S^T[key, query] = K Q^T   16 x v_mfma_f32_32x32x16_bf16 per wavefront in
//                             two independent accumulator chains (A = K from
//                             LDS, B = Q held in registers for the whole row),
//   online softmax in float32 registers: the MFMA output layout gives each
//     lane one query and 16 keys per 32-key tile, so the row max is an in-lane
//     max3 reduction plus one exchange with lane ^ 32; exp2 with sigma*log2(e)
//     folded into one FMA.  The reference max is only raised when a sub-tile's
//     max exceeds it by more than 2^8 (in exp2 units), so the rescale of the
//     output accumulators is rare; probabilities stay below 2^8.
//   P is rounded to bf16 once, and the row sum used to normalise O is taken
//     over those rounded values with v_dot2 (two per instruction), so the
//     weights the MFMA sees are normalised by their own sum; when the LSE is
//     asked for, the unrounded sum is kept beside it for that output,
//   O^T[d, query] += V^T P^T  16 MFMAs in four chains (A = V^T from LDS,
//                             B = P straight from the S^T register layout).
// Software pipeline: the S MFMAs of sub-tile t+1 are issued while the softmax
// of sub-tile t runs, so K runs one sub-tile ahead of V.  K and V both go from
// global memory straight into LDS with global_load_lds_dwordx4 (no registers):
// the K of sub-tile t+2 and the V of sub-tile t+1 are fetched during step t.
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
// Workgroups are mapped to rows XCD-aware: consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs, so row = (id % 8) * rows_per_xcd +
// id / 8 keeps consecutive query blocks of one head on one XCD, where their
// overlapping key-block lists hit the same L2.

#include "sparstar_internal.h"

#include <type_traits>

namespace sparstar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BQ = 128;            // query block
constexpr int BK = 128;            // key block
constexpr int HD = 128;            // head_dim
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;       // lazy-rescale threshold, exp2 units

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

constexpr int SUB = 64;            // keys per LDS sub-tile (half a key block)

// LDS layout (bytes): two K sub-tile buffers [64 keys][256 B], then two V^T
// sub-tile buffers [128 features][128 B].
constexpr int kKBuf = SUB * HD * 2;    // 16 KB
constexpr int kVBuf = SUB * HD * 2;    // 16 KB
constexpr int kKOff0 = 0, kVOff0 = 2 * kKBuf;
constexpr int kSmem = 2 * kKBuf + 2 * kVBuf;

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

typedef short v4s __attribute__((ext_vector_type(4)));

template <bool kDense, bool kOutBf16, bool kLse>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(AttnArgs a, int rows_per_xcd) {
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  const Geometry& g = a.g;
  const int64_t total_rows = (int64_t)g.B * g.H * g.n_q;
  const int64_t row = (int64_t)(blockIdx.x % kXcds) * rows_per_xcd + blockIdx.x / kXcds;
  if (row >= total_rows) return;  // uniform over the workgroup

  const int64_t bh = row / g.n_q;
  const int qi = (int)(row - bh * g.n_q);
  const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

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
  const float c = a.sigma * kLog2e;

  // The block lists are read-only here: read them through the scalar cache.
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  const cint_ptr rp = (cint_ptr)a.row_ptr;
  const cint_ptr ci = (cint_ptr)a.col_idx;
  // List positions fit in 32 bits: row_ptr entries are int32.
  int beg = 0, end = g.n_k;
  if (!kDense) {
    beg = rp[row];
    end = rp[row + 1];
    if (beg < 0) beg = 0;
    if ((int64_t)end > a.col_idx_len) end = (int)a.col_idx_len;
  }
  auto next_valid = [&](int p) -> int {
    if (!kDense) {
      while (p < end) {
        const int j = ci[p];
        if (j >= 0 && j < g.n_k) break;
        ++p;
      }
    }
    return p;
  };
  // A sub-tile: half h of key block j at list position p; len real keys (1..64).
  struct Sub {
    int p, j, h, len;
  };
  auto make_sub = [&](int p, int h) -> Sub {
    Sub s;
    s.p = p;
    s.h = h;
    s.j = p < end ? (kDense ? (int)p : ci[p]) : 0;
    s.len = p < end ? min(SUB, (int)g.L_k - s.j * BK - h * SUB) : 0;
    return s;
  };
  auto advance = [&](const Sub& s) -> Sub {
    if (s.p >= end) return s;
    if (s.h == 0 && (int)g.L_k - s.j * BK > SUB) return make_sub(s.p, 1);
    return make_sub(next_valid(s.p + 1), 0);
  };

  // K and V staging (direct to LDS): wavefront w, round t (0..3) fills rows
  // 16t + 4w .. +4 of a sub-tile; lane i writes row +i/16 at physical chunk i%16.
  // K rows hold logical chunk c at physical chunk c ^ (row & 15); V rows at
  // c ^ (2 * (row & 7)).
  const int st_row0 = 4 * wave + (lane >> 4);  // row in round 0; round t adds 16t
  // In-head byte offsets fit in 32 bits (the host routes larger layouts elsewhere).
  const uint32_t ks_b = (uint32_t)a.ks_t * 2u, vs_b = (uint32_t)a.vs_t * 2u;  // bytes per key
  const uint32_t k_thr = (uint32_t)st_row0 * ks_b + (uint32_t)(((lane & 15) ^ (st_row0 & 15)) * 16);
  const uint32_t v_thr = (uint32_t)st_row0 * vs_b + (uint32_t)(((lane & 15) ^ (2 * (st_row0 & 7))) * 16);

  // LDS read offsets.  K: row kt*32 + l32, logical chunk 2ks + hl, physical chunk
  // (2ks + hl) ^ (row & 15) = 2ks ^ (hl ^ (l32 & 15)); kt adds 32 rows.
  const uint32_t k_row = l32 * (HD * 2), k_sw = hl ^ (l32 & 15);
  // V^T operand by transposing reads.  Lane L = 16g + m points at key
  // 16ks + 8r + 4(g >> 1) + (m >> 2) (r = 0, 1 for the two reads of a step) and
  // features 32dt + 16(g & 1) + 4(m & 3) .. +4: chunk 4dt + cc, cc = 2(g & 1) + (m & 3) / 2,
  // byte 8 (m & 1) in it; physical chunk (4dt + cc) ^ 2kr with kr = 4(g >> 1) + (m >> 2)
  // (keys 16ks + 8r + kr share row & 7), i.e. (cc ^ 2kr) ^ 4dt.
  uint32_t v_tr[HD / 32];
  {
    const int g16 = lane >> 4, m16 = lane & 15;
    const int kr = 4 * (g16 >> 1) + (m16 >> 2);
    const int cx = (2 * (g16 & 1) + ((m16 & 3) >> 1)) ^ (2 * kr);
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
      v_tr[dt] = (uint32_t)(kr * (HD * 2) + ((cx ^ (4 * dt)) << 4) + 8 * (m16 & 1));
  }

  // Rows past the end of a partial sub-tile read row 0 instead: their scores are
  // masked to -inf, so their probabilities are exactly 0 and the P.V product adds
  // 0 times a real, finite V row.
  auto load_tile = [&](const char* base, uint32_t stride_b, uint32_t thr, const Sub& s, int off, bool is_v) {
    const char* blk = base + (uint32_t)(s.j * BK + s.h * SUB) * stride_b;
    const uint32_t ldsb = (uint32_t)(uintptr_t)(smem + off + 4 * wave * (HD * 2));
    if (s.len == SUB) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(blk + t * 16u * stride_b + thr),
                                         reinterpret_cast<__attribute__((address_space(3))) void*>(
                                             ldsb + t * 16 * (HD * 2)),
                                         16, 0, 0);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + st_row0;
        const uint32_t src_off = r < s.len ? t * 16u * stride_b + thr
                                           : (uint32_t)(((lane & 15) ^ (is_v ? 2 * (r & 7) : (r & 15))) * 16);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(blk + src_off),
                                         reinterpret_cast<__attribute__((address_space(3))) void*>(
                                             ldsb + t * 16 * (HD * 2)),
                                         16, 0, 0);
      }
    }
  };
  auto load_k = [&](const Sub& s, int off) { load_tile(kbase, ks_b, k_thr, s, off, false); };
  auto load_v = [&](const Sub& s, int off) { load_tile(vbase, vs_b, v_thr, s, off, true); };
  auto k_frag = [&](int koff, int kt, int ks) -> bf16x8 {
    return as_bf16x8(*reinterpret_cast<const uint4*>(smem + koff + kt * 32 * (HD * 2) + k_row +
                                                      (((2 * ks) ^ k_sw) << 4)));
  };
  auto v_frag = [&](int voff, int dt, int ks) -> bf16x8 {
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const uint32_t base = (uint32_t)(uintptr_t)(smem + voff + ks * 16 * (HD * 2)) + v_tr[dt];
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(base));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(base + 8 * (HD * 2)));
    bf16x8 r;
    __builtin_memcpy(&r, &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
    return r;
  };
  // S^T of one sub-tile from K buffer koff (two 32-key tiles, eight 16-feature steps).
  auto compute_s = [&](int koff, f32x16 (&s)[SUB / 32]) {
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks)
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt) {
        const bf16x8 kf = k_frag(koff, kt, ks);
        if (ks == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], z, 0, 0, 0);
        } else {
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kt], 0, 0, 0);
        }
      }
  };

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // S of the current and the next sub-tile; the two arrays swap roles every step.
  f32x16 sA[SUB / 32], sB[SUB / 32];

  // Prologue: sub-tiles c0 (K and V), c1 (K) in flight; S of c0.
  Sub cur = make_sub(next_valid(beg), 0);
  Sub nxt = advance(cur);
  if (cur.p < end) {
    load_k(cur, kKOff0);
    load_v(cur, kVOff0);
    if (nxt.p < end) load_k(nxt, kKOff0 + kKBuf);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (cur.p < end) compute_s(kKOff0, sA);
  __syncthreads();

  // One pipeline step for the sub-tile with sequence parity PAR: its K was in
  // K buffer PAR, its V is in V buffer PAR; the next sub-tile's K is in K buffer
  // PAR ^ 1.  During the step: the K of the sub-tile after next goes to K buffer
  // PAR, the next V to V buffer PAR ^ 1.
  auto step = [&](auto par) {
    constexpr int PAR = decltype(par)::value;
    constexpr int kOffCur = kKOff0 + PAR * kKBuf, kOffNxt = kKOff0 + (PAR ^ 1) * kKBuf;
    constexpr int vOffCur = kVOff0 + PAR * kVBuf, vOffNxt = kVOff0 + (PAR ^ 1) * kVBuf;
    f32x16(&s_cur)[SUB / 32] = PAR == 0 ? sA : sB;
    f32x16(&s_nxt)[SUB / 32] = PAR == 0 ? sB : sA;
    const Sub nn = advance(nxt);
    if (nn.p < end) load_k(nn, kOffCur);
    if (nxt.p < end) load_v(nxt, vOffNxt);

    // Softmax statistics of the current sub-tile.
    if (cur.len < SUB) {
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key >= cur.len) s_cur[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = (mx - m_run) * c > kTau;
    if (__any(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l *= alpha;
      if (kLse) l_exact *= alpha;
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;

    // Interleaved: S of the next sub-tile (MFMA) with P of this one (VALU).
    compute_s(kOffNxt, s_nxt);
    bf16x8 pf[SUB / 16];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        union {
          bf16x8 v;
          bf16x2 q[4];
        } pu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f32x2 f;
          f[0] = __builtin_amdgcn_exp2f(fmaf(s_cur[kt][8 * hh + 2 * e], c, -mc));
          f[1] = __builtin_amdgcn_exp2f(fmaf(s_cur[kt][8 * hh + 2 * e + 1], c, -mc));
          if (kLse) l_exact += f[0] + f[1];
          pu.q[e] = __builtin_convertvector(f, bf16x2);
          if (kt == 0) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pu.q[e], ones, rs0, false);
          else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pu.q[e], ones, rs1, false);
        }
        pf[kt * 2 + hh] = pu.v;
      }
    // 16 x (1 K read, 1 MFMA, 6 VALU of the softmax).
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
    }
    l += rs0 + rs1;

    // O^T += V^T P^T: 16 (dt, ks) steps, two transposing reads each.
#pragma unroll
    for (int ks = 0; ks < SUB / 16; ++ks)
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vOffCur, dt, ks), pf[ks], o[dt], 0, 0, 0);

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

  // Epilogue: the two lanes of a query hold partial row sums of disjoint keys.
  const float l_tot = l + __shfl_xor(l, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float le = kLse ? l_exact + __shfl_xor(l_exact, 32) : 0.f;
  if (q_valid) {
    if (kOutBf16) {
      __bf16* orow = static_cast<__bf16*>(a.out) + bi * a.os_b + hi * a.os_h + qrow * a.os_t;
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
      float* orow = static_cast<float*>(a.out) + bi * a.os_b + hi * a.os_h + qrow * a.os_t;
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float4 v4 = make_float4(o[dt][gq * 4] * inv, o[dt][gq * 4 + 1] * inv, o[dt][gq * 4 + 2] * inv,
                                  o[dt][gq * 4 + 3] * inv);
          *reinterpret_cast<float4*>(orow + dt * 32 + gq * 8 + hl * 4) = v4;
        }
    }
    if (kLse && hl == 0) a.lse[bh * g.L_q + qrow] = le > 0.f ? m_run * a.sigma + __logf(le) : -INFINITY;
  }
}

template <bool kDense, bool kOutBf16, bool kLse>
void launch(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.n_q;
  const int rows_per_xcd = (int)((rows + kXcds - 1) / kXcds);
  const int64_t grid = (int64_t)rows_per_xcd * kXcds;
  hipLaunchKernelGGL((attn_mfma_kernel<kDense, kOutBf16, kLse>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                     rows_per_xcd);
}

template <bool kDense, bool kOutBf16>
void launch2(const AttnArgs& a, hipStream_t s) {
  if (a.lse) launch<kDense, kOutBf16, true>(a, s);
  else launch<kDense, kOutBf16, false>(a, s);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.g.D != HD || a.g.b != BQ || a.dtype != 0) return hipErrorInvalidValue;
  const bool dense = a.row_ptr == nullptr;
  const bool ob = a.out_dtype == 0;
  if (dense) ob ? launch2<true, true>(a, s) : launch2<true, false>(a, s);
  else ob ? launch2<false, true>(a, s) : launch2<false, false>(a, s);
  return hipGetLastError();
}

}  // namespace sparstar
