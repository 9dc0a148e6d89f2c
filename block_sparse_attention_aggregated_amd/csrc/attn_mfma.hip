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
// While a sub-tile is computed, the next one is fetched: K straight into the
// other LDS buffer with global_load_lds_dwordx4 (no registers), V into 16
// registers, written to LDS transposed (v_perm 4 x 8 transposes) after the
// P.V product.  V keys of each 16-key group are permuted so that a lane's
// eight P values (keys 8*(r/4) + 4*half + r%4 of the S^T layout) meet the
// matching eight V values in one 16-byte LDS read.  K rows (256 bytes) and
// V^T rows (128 bytes) have XOR-swizzled 16-byte chunks: the MFMA operand
// reads are free of bank conflicts without padding.  One barrier per sub-tile.
// The block lists are read through the scalar cache.
//
// Workgroups are mapped to rows XCD-aware: consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs, so row = (id % 8) * rows_per_xcd +
// id / 8 keeps consecutive query blocks of one head on one XCD, where their
// overlapping key-block lists hit the same L2.

#include "sparstar_internal.h"

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

// Chunk swizzles (16-byte chunks).  K rows are 256 bytes (16 chunks), V^T rows
// 128 bytes (8 chunks of one 64-key sub-tile).
__device__ inline int k_chunk(int row, int chunk) { return chunk ^ (row & 15); }
__device__ inline int v_chunk(int d, int chunk) { return chunk ^ (((d >> 1) ^ (d >> 4)) & 7); }

template <bool kDense, bool kOutBf16, bool kLse>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(AttnArgs a, int rows_per_xcd) {
  // Two buffers of one 64-key sub-tile each: K [64 keys][128 features] and
  // V^T [128 features][64 key positions].
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][SUB * HD];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][HD * SUB];

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
  float m_run = -INFINITY, l = 0.f, l_exact = 0.f;  // l: sum of the bf16-rounded P; l_exact: unrounded
  const float c = a.sigma * kLog2e;

  // The block lists are read-only here: read them through the scalar cache.
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  const cint_ptr rp = (cint_ptr)a.row_ptr;
  const cint_ptr ci = (cint_ptr)a.col_idx;
  int64_t beg = 0, end = g.n_k;
  if (!kDense) {
    beg = rp[row];
    end = rp[row + 1];
    if (beg < 0) beg = 0;
    if (end > a.col_idx_len) end = a.col_idx_len;
  }
  auto col = [&](int64_t p) -> int { return kDense ? (int)p : ci[p]; };
  auto next_valid = [&](int64_t p) -> int64_t {
    if (!kDense) {
      while (p < end) {
        const int j = ci[p];
        if (j >= 0 && j < g.n_k) break;
        ++p;
      }
    }
    return p;
  };
  // Real keys in sub-tile h of block j (<= 0: the sub-tile is empty).
  auto sub_len = [&](int j, int h) -> int {
    return (int)min<int64_t>(SUB, g.L_k - (int64_t)j * BK - (int64_t)h * SUB);
  };

  // K staging (direct to LDS): wavefront w, round t fills rows 16t + 4w .. +4 of a
  // sub-tile; lane i writes row +i/16, physical chunk i%16, i.e. logical chunk
  // (i%16) ^ (row%16) of that key.
  const int k_row_in_round = 4 * wave + (lane >> 4);
  const int k_lchunk = (lane & 15) ^ (k_row_in_round & 15);
  const int64_t k_thr = ((int64_t)k_row_in_round * a.ks_t + k_lchunk * 8) * 2;   // bytes
  const int64_t k_round = (int64_t)16 * a.ks_t * 2;                                  // bytes per round
  // V staging (registers): keys 4*kg .. +4 of the sub-tile, features 8*fg .. +8.
  const int fg = tid & 15, kg = tid >> 4;
  const int64_t v_thr = ((int64_t)(4 * kg) * a.vs_t + fg * 8) * 2;                   // bytes
  const int v_s = kg >> 2, v_a = (kg & 3) >> 1, v_hh = kg & 1;
  uint4 vst[4];

  auto issue_loads = [&](int j, int h, int buf) {
    const int len = sub_len(j, h);
    const int64_t key0 = (int64_t)j * BK + h * SUB;
    const char* kblk = kbase + key0 * a.ks_t * 2;
    const char* vblk = vbase + key0 * a.vs_t * 2;
    char* kdst = reinterpret_cast<char*>(&Ks[buf][0]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 16 * t + k_row_in_round;
      const char* src = kblk + (r < len ? t * k_round + k_thr : (int64_t)(lane & 15) * 16);
      char* dst = kdst + (16 * t + 4 * wave) * (HD * 2);  // wave-uniform LDS base of this round
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           (uint32_t)(uintptr_t)dst),
                                       16, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 4 * kg + e;
      vst[e] = ld16(vblk + (key < len ? (int64_t)e * a.vs_t * 2 + v_thr : (int64_t)fg * 16));
    }
  };

  auto store_v = [&](int len, int buf) {
    if (len < SUB) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * kg + e >= len) vst[e] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint4 x = vst[e];
        w[e] = (dd >> 1) == 0 ? x.x : (dd >> 1) == 1 ? x.y : (dd >> 1) == 2 ? x.z : x.w;
      }
      uint2 outv;
      outv.x = __builtin_amdgcn_perm(w[1], w[0], sel);
      outv.y = __builtin_amdgcn_perm(w[3], w[2], sel);
      const int d = fg * 8 + dd;
      *reinterpret_cast<uint2*>(&Vt[buf][d * SUB + v_chunk(d, 2 * v_s + v_hh) * 8 + 4 * v_a]) = outv;
    }
  };

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  int64_t p = next_valid(beg);
  int h = 0, buf = 0;
  if (p < end) {
    issue_loads(col(p), 0, 0);
    store_v(sub_len(col(p), 0), 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

#pragma unroll 1
  while (p < end) {
    const int j = col(p);
    const int len = sub_len(j, h);
    // Next sub-tile: the second half of this block if it has keys, else the next block.
    int64_t pn = p;
    int hn = 1;
    if (h == 1 || sub_len(j, 1) <= 0) {
      pn = next_valid(p + 1);
      hn = 0;
    }
    const bool has_next = pn < end;
    int jn = 0;
    if (has_next) {
      jn = col(pn);
      issue_loads(jn, hn, buf ^ 1);
    }

    // S^T = K Q^T: two independent 32-key tiles, eight steps of 16 features.
    f32x16 s[SUB / 32];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
      bf16x8 kf[SUB / 32];
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt) {
        const int r = kt * 32 + l32;
        kf[kt] = as_bf16x8(ld16(&Ks[buf][r * HD + k_chunk(r, ks * 2 + hl) * 8]));
      }
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt) {
        if (ks == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt], qf[ks], z, 0, 0, 0);
        } else {
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt], qf[ks], s[kt], 0, 0, 0);
        }
      }
    }
    if (len < SUB) {
#pragma unroll
      for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key >= len) s[kt][r] = -INFINITY;
        }
    }
    // Sub-tile max, lazy update of the reference max.
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < SUB / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
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

    // P = exp2(s*c - m*c) in bf16, laid out as the B operand of the P.V MFMA; row
    // sums over the rounded values with v_dot2.
    bf16x8 pf[SUB / 16];
    float rs[SUB / 32];
#pragma unroll
    for (int kt = 0; kt < SUB / 32; ++kt) {
      rs[kt] = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        union {
          bf16x8 v;
          bf16x2 q[4];
        } pu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f32x2 f;
          f[0] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * hh + 2 * e], c, -mc));
          f[1] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * hh + 2 * e + 1], c, -mc));
          if (kLse) l_exact += f[0] + f[1];
          pu.q[e] = __builtin_convertvector(f, bf16x2);
          rs[kt] = __builtin_amdgcn_fdot2_f32_bf16(pu.q[e], ones, rs[kt], false);
        }
        pf[kt * 2 + hh] = pu.v;
      }
    }
    l += rs[0] + rs[1];

    // O^T += V^T P^T: four independent 32-feature tiles, four steps of 16 keys.
#pragma unroll
    for (int ks = 0; ks < SUB / 16; ++ks) {
      bf16x8 vf[HD / 32];
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) {
        const int d = dt * 32 + l32;
        vf[dt] = as_bf16x8(ld16(&Vt[buf][d * SUB + v_chunk(d, ks * 2 + hl) * 8]));
      }
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt], pf[ks], o[dt], 0, 0, 0);
    }

    if (has_next) store_v(sub_len(jn, hn), buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // direct-to-LDS K writes of the next sub-tile have landed
    __syncthreads();
    p = pn;
    h = hn;
    buf ^= 1;
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
