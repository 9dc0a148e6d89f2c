// K3/K4: block-sparse (and dense) attention forward on gfx950 bf16 MFMA.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Forward-Only Sparse Execution" and "Complexity and Scope": each
// query block visits only the key blocks of its list, so the work scales with
// the retained fraction of blocks; softmax over the real keys of those blocks.
//
// Shape: bf16 Q/K/V, head_dim 128, 128-token query and key blocks.
// One workgroup (4 wavefronts) per query block; wavefront w owns queries
// 32w .. 32w+31 of the block.  Per key block:
//   S^T[key, query] = K Q^T   32 x v_mfma_f32_32x32x16_bf16 per wavefront
//                             (A = K from LDS, B = Q held in registers),
//   online softmax in float32 registers: the MFMA output layout gives each
//     lane one query and 16 keys per 32-key tile, so the row max is an in-lane
//     reduction plus one exchange with lane ^ 32, and exp2 with sigma*log2(e)
//     folded into a single FMA,
//   O^T[d, query] += V^T P^T  32 MFMAs (A = V^T from LDS, B = P in registers,
//                             converted to bf16 straight from the S^T layout).
// V is transposed while it is staged into LDS (8 x 8 register transposes with
// v_perm), with the keys of every 16-key group permuted so that a lane's
// eight P values (keys 8*(r/4) + 4*half + r%4 of the S^T layout) meet the
// matching eight V values in one 16-byte LDS read.  LDS rows are padded by 16
// bytes against bank conflicts.
//
// Workgroups are mapped to rows XCD-aware: consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs, so row = (id % 8) * rows_per_xcd +
// id / 8 keeps consecutive query blocks of one head on one XCD, where their
// overlapping key-block lists hit the same L2.

#include "sparstar_internal.h"

namespace sparstar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BQ = 128;            // query block
constexpr int BK = 128;            // key block
constexpr int HD = 128;            // head_dim
constexpr int KS = HD + 8;         // K tile row stride in LDS (bf16 elements)
constexpr int VS = BK + 8;         // V^T tile row stride in LDS
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <bool kDense, bool kOutBf16>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(AttnArgs a, int rows_per_xcd) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[BK * KS];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[HD * VS];

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
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + bi * a.ks_b + hi * a.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + bi * a.vs_b + hi * a.vs_h;

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
  float m = -INFINITY, l = 0.f;
  const float c = a.sigma * kLog2e;

  int64_t beg = 0, end = g.n_k;
  if (!kDense) {
    beg = a.row_ptr[row];
    end = a.row_ptr[row + 1];
    if (beg < 0) beg = 0;
    if (end > a.col_idx_len) end = a.col_idx_len;
  }

  // Staging roles.
  const int ld_ch = tid & 15;          // 16-byte chunk of a 256-byte row
  const int ld_row = tid >> 4;         // 0..15
  const int vg = tid >> 4;             // V: group of 8 keys (LDS positions 8*vg .. +8)
  const int v_s16 = vg >> 1, v_h = vg & 1;

#pragma unroll 1
  for (int64_t p = beg; p < end; ++p) {
    const int j = kDense ? (int)p : a.col_idx[p];
    if (j < 0 || j >= g.n_k) continue;  // same j for the whole workgroup
    const int kv_len = (int)min<int64_t>(BK, g.L_k - (int64_t)j * BK);
    const int64_t key0 = (int64_t)j * BK;

    __syncthreads();  // previous tile fully consumed
    // K tile: rows 16*it + ld_row, chunk ld_ch.
#pragma unroll
    for (int it = 0; it < BK / 16; ++it) {
      const int r = it * 16 + ld_row;
      const uint4 v = r < kv_len ? ld16(kbase + (key0 + r) * a.ks_t + ld_ch * 8) : make_uint4(0, 0, 0, 0);
      st16(&Ks[r * KS + ld_ch * 8], v);
    }
    // V tile, transposed: this thread loads 8 keys x 8 features (features 8*ld_ch .. +8) and
    // writes 8 rows of V^T (one per feature), 8 consecutive LDS key positions each.
    {
      uint4 vr[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int key = v_s16 * 16 + (jj >> 2) * 8 + v_h * 4 + (jj & 3);
        vr[jj] = key < kv_len ? ld16(vbase + (key0 + key) * a.vs_t + ld_ch * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint4 x = vr[jj];
          w[jj] = (dd >> 1) == 0 ? x.x : (dd >> 1) == 1 ? x.y : (dd >> 1) == 2 ? x.z : x.w;
        }
        uint4 outv;
        outv.x = __builtin_amdgcn_perm(w[1], w[0], sel);
        outv.y = __builtin_amdgcn_perm(w[3], w[2], sel);
        outv.z = __builtin_amdgcn_perm(w[5], w[4], sel);
        outv.w = __builtin_amdgcn_perm(w[7], w[6], sel);
        st16(&Vt[(ld_ch * 8 + dd) * VS + vg * 8], outv);
      }
    }
    __syncthreads();

    // S^T = K Q^T over 4 tiles of 32 keys.
    f32x16 s[BK / 32];
#pragma unroll
    for (int kt = 0; kt < BK / 32; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const bf16x8 kf = as_bf16x8(ld16(&Ks[(kt * 32 + l32) * KS + ks * 16 + hl * 8]));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kt], 0, 0, 0);
      }
    }
    if (kv_len < BK) {
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key >= kv_len) s[kt][r] = -INFINITY;
        }
    }
    // Online softmax (raw logits; sigma*log2(e) folded into the exponent).
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    const float mc = m_new * c;
    float rs = 0.f;
    bf16x8 pf[BK / 16];
#pragma unroll
    for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -mc));
        rs += pv;
        pf[kt * 2 + (r >> 3)][r & 7] = (__bf16)pv;
      }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // O^T += V^T P^T over 8 steps of 16 keys.
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const bf16x8 vf = as_bf16x8(ld16(&Vt[(dt * 32 + l32) * VS + ks * 16 + hl * 8]));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[dt], 0, 0, 0);
      }
  }

  // Epilogue: the two lanes of a query hold partial row sums of disjoint keys.
  const float l_tot = l + __shfl_xor(l, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
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
    if (a.lse && hl == 0)
      a.lse[bh * g.L_q + qrow] = l_tot > 0.f ? m * a.sigma + __logf(l_tot) : -INFINITY;
  }
}

template <bool kDense, bool kOutBf16>
void launch(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.n_q;
  const int rows_per_xcd = (int)((rows + kXcds - 1) / kXcds);
  const int64_t grid = (int64_t)rows_per_xcd * kXcds;
  hipLaunchKernelGGL((attn_mfma_kernel<kDense, kOutBf16>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                     rows_per_xcd);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.g.D != HD || a.g.b != BQ || a.dtype != 0) return hipErrorInvalidValue;
  const bool dense = a.row_ptr == nullptr;
  const bool ob = a.out_dtype == 0;
  if (dense) ob ? launch<true, true>(a, s) : launch<true, false>(a, s);
  else ob ? launch<false, true>(a, s) : launch<false, false>(a, s);
  return hipGetLastError();
}

}  // namespace sparstar
