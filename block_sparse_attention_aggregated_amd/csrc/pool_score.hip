// Block mean-pooling and aggregated-QK block scores.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Original-order block partition": contiguous blocks of b tokens,
// the final partial block zero-padded and averaged over the nominal b; and
// "Per-head aggregated query-key score": one score per (query block, key
// block) pair and head, here sigma * <qbar_i, kbar_j>.
//
// pool_kernel is a pure HBM stream: each workgroup reads one block of b
// tokens x D features (32 KB for bf16, b = D = 128) with 16-byte loads, each
// 16-lane group covering one 256-byte token row, and reduces the rows in
// float32 through cross-lane shuffles and a small LDS exchange.
// score_kernel is a small float32 GEMM per (batch, head): 64 x 64 output
// tiles, K = D, operands staged through LDS, 4 x 4 outputs per thread.

#include "sparstar_internal.h"

namespace sparstar {
namespace {

constexpr int kPoolThreads = 256;

__device__ inline void load16_to_f32(const __bf16* src, float* dst8) {
  const uint4 raw = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst8[2 * i] = __uint_as_float(w[i] << 16);
    dst8[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline void load16_to_f32(const float* src, float* dst4) {
  const float4 raw = *reinterpret_cast<const float4*>(src);
  dst4[0] = raw.x; dst4[1] = raw.y; dst4[2] = raw.z; dst4[3] = raw.w;
}

// One workgroup per (batch, head, block), query blocks first then key blocks.
// VEC elements per 16-byte load; CH = D / VEC column chunks; G = 256 / CH row groups.
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolScoreArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CH = D / VEC;
  constexpr int G = kPoolThreads / CH;
  __shared__ float red[G][D + 4];

  const Geometry& g = a.g;
  const int64_t per_bh = (int64_t)g.n_q + g.n_k;
  const int64_t wid = blockIdx.x;
  const int64_t bh = wid / per_bh;
  int64_t j = wid - bh * per_bh;
  const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);
  const bool is_q = j < g.n_q;
  if (!is_q) j -= g.n_q;
  const T* base;
  int64_t ts, L;
  float* dst;
  if (is_q) {
    base = static_cast<const T*>(a.q) + bi * a.qs_b + hi * a.qs_h;
    ts = a.qs_t;
    L = g.L_q;
    dst = a.q_pool + (bh * g.n_q + j) * D;
  } else {
    base = static_cast<const T*>(a.k) + bi * a.ks_b + hi * a.ks_h;
    ts = a.ks_t;
    L = g.L_k;
    dst = a.k_pool + (bh * g.n_k + j) * D;
  }
  const int64_t t0 = j * g.b;
  const int n_tok = (int)min<int64_t>(g.b, L - t0);

  const int c = threadIdx.x % CH, grp = threadIdx.x / CH;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  // b / G rows per thread (8 for bf16 at b = D = 128); all loads issued first.
  constexpr int kMaxRows = 128 / G > 0 ? 128 / G : 1;
  float vals[kMaxRows][VEC];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    const int t = grp + r * G;
    if (t < n_tok) {
      load16_to_f32(base + (t0 + t) * ts + c * VEC, vals[r]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) vals[r][e] = 0.f;
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += vals[r][e];

#pragma unroll
  for (int e = 0; e < VEC; ++e) red[grp][c * VEC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < G; ++r) s += red[r][threadIdx.x];
    dst[threadIdx.x] = s / (float)g.b;
  }
}

// S[bh, i, j] = sigma * sum_d qp[bh, i, d] * kp[bh, j, d].  Tile 64 x 64, 256 threads,
// 4 x 4 outputs per thread; the D dimension is staged in chunks of 32 through LDS.
constexpr int kTile = 64, kDc = 32;

template <int D>
__global__ __launch_bounds__(256) void score_kernel(PoolScoreArgs a, int tiles_i, int tiles_j) {
  __shared__ float As[kDc][kTile + 4];
  __shared__ float Bs[kDc][kTile + 4];
  const Geometry& g = a.g;
  const int64_t tile = blockIdx.x;
  const int64_t per_bh = (int64_t)tiles_i * tiles_j;
  const int64_t bh = tile / per_bh;
  const int rem = (int)(tile - bh * per_bh);
  const int ti = rem / tiles_j, tj = rem - (rem / tiles_j) * tiles_j;
  const int i0 = ti * kTile, j0 = tj * kTile;
  const float* qp = a.q_pool + bh * g.n_q * D;
  const float* kp = a.k_pool + bh * g.n_k * D;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;

  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[r][s] = 0.f;

  // Loader: 64 rows x 32 columns per operand = 512 float4; 2 per thread per operand.
  for (int d0 = 0; d0 < D; d0 += kDc) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = threadIdx.x + u * 256;
      const int row = idx / (kDc / 4), col4 = idx % (kDc / 4);
      float4 qa = make_float4(0.f, 0.f, 0.f, 0.f), kb = qa;
      if (i0 + row < g.n_q) qa = *reinterpret_cast<const float4*>(qp + (int64_t)(i0 + row) * D + d0 + col4 * 4);
      if (j0 + row < g.n_k) kb = *reinterpret_cast<const float4*>(kp + (int64_t)(j0 + row) * D + d0 + col4 * 4);
      As[col4 * 4 + 0][row] = qa.x; As[col4 * 4 + 1][row] = qa.y;
      As[col4 * 4 + 2][row] = qa.z; As[col4 * 4 + 3][row] = qa.w;
      Bs[col4 * 4 + 0][row] = kb.x; Bs[col4 * 4 + 1][row] = kb.y;
      Bs[col4 * 4 + 2][row] = kb.z; Bs[col4 * 4 + 3][row] = kb.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int d = 0; d < kDc; ++d) {
      const float4 x = *reinterpret_cast<const float4*>(&As[d][ty * 4]);
      const float4 y = *reinterpret_cast<const float4*>(&Bs[d][tx * 4]);
      const float xa[4] = {x.x, x.y, x.z, x.w}, ya[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[r][s] = fmaf(xa[r], ya[s], acc[r][s]);
    }
    __syncthreads();
  }
  float* S = a.scores + bh * (int64_t)g.n_q * g.n_k;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + ty * 4 + r;
    if (i >= g.n_q) continue;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int j = j0 + tx * 4 + s;
      if (j < g.n_k) S[(int64_t)i * g.n_k + j] = a.sigma * acc[r][s];
    }
  }
}

template <typename T, int D>
hipError_t launch_pool(const PoolScoreArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.g.B * a.g.H * ((int64_t)a.g.n_q + a.g.n_k);
  if (blocks > 0) hipLaunchKernelGGL((pool_kernel<T, D>), dim3((unsigned)blocks), dim3(kPoolThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_score(const PoolScoreArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.g.b > 128) return hipErrorInvalidValue;  // pool_kernel holds up to 128 rows per workgroup
  if (a.dtype == 0)
    e = a.g.D == 128 ? launch_pool<__bf16, 128>(a, s) : launch_pool<__bf16, 64>(a, s);
  else
    e = a.g.D == 128 ? launch_pool<float, 128>(a, s) : launch_pool<float, 64>(a, s);
  if (e != hipSuccess) return e;
  const int ti = (a.g.n_q + kTile - 1) / kTile, tj = (a.g.n_k + kTile - 1) / kTile;
  const int64_t tiles = (int64_t)a.g.B * a.g.H * ti * tj;
  if (tiles > 0) {
    if (a.g.D == 128)
      hipLaunchKernelGGL(score_kernel<128>, dim3((unsigned)tiles), dim3(256), 0, s, a, ti, tj);
    else
      hipLaunchKernelGGL(score_kernel<64>, dim3((unsigned)tiles), dim3(256), 0, s, a, ti, tj);
  }
  return hipGetLastError();
}

}  // namespace sparstar
