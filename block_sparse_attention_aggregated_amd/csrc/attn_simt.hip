// Float32 path: block-sparse (and dense) attention forward for float32
// inputs and for the shapes the MFMA kernel does not cover (head_dim 64).  Same
// semantics as the MFMA kernel ("SparSTAR: Sparse Attention for SpaceTime
// AutoRegressive Video Synthesis", section 5
// "Forward-Only Sparse Execution"): every query of block i attends, with a
// softmax over real keys only, to the key blocks listed for row i.
//
// One workgroup per query block, one thread per query.  Keys and values are
// staged through LDS in float32, 32 keys at a time, and every thread runs an
// online softmax over them in float32 with accurate exp.

#include "sparstar_internal.h"

namespace sparstar {
namespace {

constexpr int kChunk = 32;

template <typename T>
__device__ inline float to_f32(T x);
template <>
__device__ inline float to_f32<float>(float x) { return x; }
template <>
__device__ inline float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T, int D, bool kDense, typename OutT>
__global__ __launch_bounds__(256) void attn_simt_kernel(AttnArgs a) {
  // Unpadded rows aligned to 16 bytes: every thread reads the same row element at
  // the same time (a broadcast, free of bank conflicts), so the rows need no pad,
  // and the reads go four features at a time (2.3x faster than padded rows read
  // one feature at a time, on the tiny float32 workload).
  __shared__ __attribute__((aligned(16))) float Kc[kChunk][D];
  __shared__ __attribute__((aligned(16))) float Vc[kChunk][D];
  const Geometry& g = a.g;
  const int64_t row = blockIdx.x;
  const int64_t bh = row / g.n_q;
  const int qi = (int)(row - bh * g.n_q);
  const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);
  const int t = threadIdx.x;  // query within the block
  const int64_t qrow = (int64_t)qi * g.b + t;
  const bool q_valid = t < g.b && qrow < g.L_q;

  const T* qb = static_cast<const T*>(a.q) + bi * a.qs_b + hi * a.qs_h;
  const T* kb = static_cast<const T*>(a.k) + bi * a.ks_b + hi * a.ks_h;
  const T* vb = static_cast<const T*>(a.v) + bi * a.vs_b + hi * a.vs_h;

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = q_valid ? to_f32(qb[qrow * a.qs_t + d]) : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int64_t beg = 0, end = g.n_k;
  if (!kDense) {
    beg = a.row_ptr[row];
    end = a.row_ptr[row + 1];
    if (beg < 0) beg = 0;
    if (end > a.col_idx_len) end = a.col_idx_len;
  }
#pragma unroll 1
  for (int64_t p = beg; p < end; ++p) {
    const int j = kDense ? (int)p : a.col_idx[p];
    if (j < 0 || j >= g.n_k) continue;
    const int64_t key0 = (int64_t)j * g.b;
    const int kv_len = (int)min<int64_t>(g.b, g.L_k - key0);
#pragma unroll 1
    for (int c0 = 0; c0 < kv_len; c0 += kChunk) {
      const int n = min(kChunk, kv_len - c0);
      __syncthreads();
      for (int idx = t; idx < kChunk * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        const bool ok = r < n;
        Kc[r][d] = ok ? to_f32(kb[(key0 + c0 + r) * a.ks_t + d]) : 0.f;
        Vc[r][d] = ok ? to_f32(vb[(key0 + c0 + r) * a.vs_t + d]) : 0.f;
      }
      __syncthreads();
      float sc[kChunk];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(q[d], Kc[r][d], acc);
        sc[r] = r < n ? acc * a.sigma : -INFINITY;
        mx = fmaxf(mx, sc[r]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        const float pr = expf(sc[r] - m_new);
        l += pr;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pr, Vc[r][d], o[d]);
      }
      m = m_new;
    }
  }
  if (!q_valid) return;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  OutT* orow = static_cast<OutT*>(a.out) + bi * a.os_b + hi * a.os_h + qrow * a.os_t;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = (OutT)(o[d] * inv);
  if (a.lse) a.lse[bh * g.L_q + qrow] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <typename T, int D, typename OutT>
void launch3(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.n_q;
  if (a.row_ptr)
    hipLaunchKernelGGL((attn_simt_kernel<T, D, false, OutT>), dim3((unsigned)rows), dim3(a.g.b), 0, s, a);
  else
    hipLaunchKernelGGL((attn_simt_kernel<T, D, true, OutT>), dim3((unsigned)rows), dim3(a.g.b), 0, s, a);
}

template <typename T, int D>
void launch2(const AttnArgs& a, hipStream_t s) {
  if (a.out_dtype == 0) launch3<T, D, __bf16>(a, s);
  else launch3<T, D, float>(a, s);
}

}  // namespace

hipError_t launch_attn_simt(const AttnArgs& a, hipStream_t s) {
  if (a.g.b > 256) return hipErrorInvalidValue;
  if (a.dtype == 0) a.g.D == 128 ? launch2<__bf16, 128>(a, s) : launch2<__bf16, 64>(a, s);
  else a.g.D == 128 ? launch2<float, 128>(a, s) : launch2<float, 64>(a, s);
  return hipGetLastError();
}

}  // namespace sparstar
