// Block mean-pooling and aggregated-QK block scores.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Original-order block partition": contiguous blocks of b tokens,
// the final partial block zero-padded and averaged over the nominal b; and
// "Per-head aggregated query-key score": one score per (query block, key
// block) pair and head, here sigma * <qbar_i, kbar_j>.
//
// pool_kernel is a pure HBM stream: each workgroup reads one block of b
// tokens x D features (32 KB for bf16, b = D = 128) with 16-byte non-temporal loads, each
// 16-lane group covering one 256-byte token row (128 rows per pass, two passes
// at b = 256); each thread sums its rows in float32 and a small LDS exchange
// sums the row groups.
// score_kernel is a small float32 GEMM per (batch, head) on the float32
// matrix cores: 64 x 128 output tiles, K = D.

#include "sparstar_internal.h"

namespace sparstar {
namespace {

constexpr int kPoolThreads = 256;

// 16 loaded bytes as float32: eight bf16 (the high halves of float32) or four float32.
__device__ inline void to_f32x(uint4 raw, float* dst8, __bf16) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst8[2 * i] = __uint_as_float(w[i] << 16);
    dst8[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline void to_f32x(uint4 raw, float* dst4, float) {
  dst4[0] = __uint_as_float(raw.x);
  dst4[1] = __uint_as_float(raw.y);
  dst4[2] = __uint_as_float(raw.z);
  dst4[3] = __uint_as_float(raw.w);
}

// 16 bytes of a stream that is read once: a non-temporal load, so the 1.8 GB of Q
// and K passing through do not displace other lines from the Infinity Cache and
// the L2s (measured 4.5% faster for the pass at 720p than plain loads).
__device__ inline uint4 load_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(w[0], w[1], w[2], w[3]);
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
  const T* base_ptr;
  int64_t ts, L;
  float* dst;
  if (is_q) {
    base_ptr = static_cast<const T*>(a.q) + bi * a.qs_b + hi * a.qs_h;
    ts = a.qs_t;
    L = g.L_q;
    dst = a.q_pool + (bh * g.n_q + j) * D;
  } else {
    base_ptr = static_cast<const T*>(a.k) + bi * a.ks_b + hi * a.ks_h;
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

  // 128 / G rows per thread and pass (8 for bf16 at D = 128); blocks of 256 tokens
  // take two passes.  All loads of a pass are issued before any is used: every
  // lane loads a real row (rows past the end re-read the last real row) and the
  // rows past the end are then zeroed by a select, so no load sits in a branch.
  constexpr int kMaxRows = 128 / G > 0 ? 128 / G : 1;
  for (int base = 0; base < n_tok; base += 128) {
    uint4 raw[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      const int t = min(base + grp + r * G, n_tok - 1);
      raw[r] = load_stream(base_ptr + (t0 + t) * ts + c * VEC);
    }
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      float v[VEC];
      to_f32x(raw[r], v, T{});
      const bool ok = base + grp + r * G < n_tok;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += ok ? v[e] : 0.f;
    }
  }

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

// S[bh, i, j] = sigma * sum_d qp[bh, i, d] * kp[bh, j, d] on the float32 matrix
// cores (v_mfma_f32_32x32x2_f32, float32 products and sums).  A workgroup of 4
// wavefronts computes a 64 x 128 tile (query blocks x key blocks); wavefront w
// the 32 x 64 part (w >> 1, w & 1) as two MFMA tiles of 32 x 32.  The 64 pooled
// query rows and 128 key rows go through LDS 32 features at a time: coalesced
// 128-byte row segments into registers (the next chunk's loads are in flight
// while the current chunk is multiplied), then into row-padded LDS tiles.  For
// MFMA step s of a chunk, lane l supplies feature 16 (l >> 5) + s of row l & 31
// of each of its tiles (the summation order within the 2-wide MFMA step is
// free, as long as both operands use the same one), read from LDS 4 features at
// a time.
// Workgroups are placed XCD-aware: XCD x (= id mod 8) scores the heads
// bh = x, x + 8, ..., so a head's pooled rows stay in one XCD's L2.
// Output: register r of a lane holds row 8 (r >> 2) + 4 (l >> 5) + (r & 3) and
// column l & 31 of its 32 x 32 tile.
constexpr int kTileI = 64, kTileJ = 128;
constexpr int kDc = 32;           // features per chunk
constexpr int kPad = kDc + 4;     // LDS row pitch in floats (144 B: conflict-free 16-byte reads)

template <int D>
__global__ __launch_bounds__(256, 2) void score_kernel(PoolScoreArgs a, int tiles_i, int tiles_j) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int kChunks = D / kDc;
  __shared__ __attribute__((aligned(16))) float As[kTileI][kPad];
  __shared__ __attribute__((aligned(16))) float Bs[kTileJ][kPad];
  const Geometry& g = a.g;
  const int64_t per_bh = (int64_t)tiles_i * tiles_j;
  const int64_t k = blockIdx.x / kXcds;
  const int64_t bh = (k / per_bh) * kXcds + blockIdx.x % kXcds;
  if (bh >= (int64_t)g.B * g.H) return;  // uniform over the workgroup
  const int rem = (int)(k % per_bh);
  const int ti = rem / tiles_j, tj = rem - ti * tiles_j;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, hl = lane >> 5;
  const float* qp = a.q_pool + bh * g.n_q * D;
  const float* kp = a.k_pool + bh * g.n_k * D;

  // Staging: thread t moves query rows (t >> 3) + 32 m, m = 0, 1, and key rows
  // (t >> 3) + 32 m, m = 0..3, 16 bytes at feature 4 (t & 7).  Rows past the end
  // copy the last row: they only feed outputs that are not stored.
  constexpr int kMa = kTileI / 32, kMb = kTileJ / 32;
  const int sr = tid >> 3, sc = 4 * (tid & 7);
  const float* ga[kMa];
  const float* gb[kMb];
#pragma unroll
  for (int m = 0; m < kMa; ++m) ga[m] = qp + (int64_t)min(ti * kTileI + sr + 32 * m, g.n_q - 1) * D + sc;
#pragma unroll
  for (int m = 0; m < kMb; ++m) gb[m] = kp + (int64_t)min(tj * kTileJ + sr + 32 * m, g.n_k - 1) * D + sc;
  f32x4 ra[kMa], rb[kMb];
  auto gload = [&](int c) {
#pragma unroll
    for (int m = 0; m < kMa; ++m) ra[m] = *reinterpret_cast<const f32x4*>(ga[m] + c * kDc);
#pragma unroll
    for (int m = 0; m < kMb; ++m) rb[m] = *reinterpret_cast<const f32x4*>(gb[m] + c * kDc);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int m = 0; m < kMa; ++m) *reinterpret_cast<f32x4*>(&As[sr + 32 * m][sc]) = ra[m];
#pragma unroll
    for (int m = 0; m < kMb; ++m) *reinterpret_cast<f32x4*>(&Bs[sr + 32 * m][sc]) = rb[m];
  };

  f32x16 acc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;

  const int arow = (wave >> 1) * 32 + r32, brow = (wave & 1) * 64 + r32;
  gload(0);
  lstore();
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (c + 1 < kChunks) gload(c + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // features 16 hl + 4q .. +4
      const f32x4 av = *reinterpret_cast<const f32x4*>(&As[arow][16 * hl + 4 * q]);
      f32x4 bv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) bv[u] = *reinterpret_cast<const f32x4*>(&Bs[brow + 32 * u][16 * hl + 4 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[u][e], acc[u], 0, 0, 0);
    }
    if (c + 1 < kChunks) {
      __syncthreads();
      lstore();
      __syncthreads();
    }
  }

  const int i0 = ti * kTileI + (wave >> 1) * 32 + 4 * hl, j0 = tj * kTileJ + (wave & 1) * 64 + r32;
  float* S = a.scores + bh * (int64_t)g.n_q * g.n_k;
  const bool interior = (ti + 1) * kTileI <= g.n_q && (tj + 1) * kTileJ <= g.n_k;  // uniform
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = j0 + 32 * u;
    float* col = S + (int64_t)i0 * g.n_k + j;
    if (interior) {
#pragma unroll
      for (int r = 0; r < 16; ++r) col[(8 * (r >> 2) + (r & 3)) * g.n_k] = a.sigma * acc[u][r];
    } else if (j < g.n_k) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (i0 + 8 * (r >> 2) + (r & 3) < g.n_q) col[(8 * (r >> 2) + (r & 3)) * g.n_k] = a.sigma * acc[u][r];
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
  if (a.g.b > 256) return hipErrorInvalidValue;  // pool_kernel walks up to 256 rows per workgroup
  if (a.dtype == 0)
    e = a.g.D == 128 ? launch_pool<__bf16, 128>(a, s) : launch_pool<__bf16, 64>(a, s);
  else
    e = a.g.D == 128 ? launch_pool<float, 128>(a, s) : launch_pool<float, 64>(a, s);
  if (e != hipSuccess) return e;
  if (a.scores == nullptr) return hipSuccess;  // pooling only
  const int ti = (a.g.n_q + kTileI - 1) / kTileI, tj = (a.g.n_k + kTileJ - 1) / kTileJ;
  // XCD-aware grid: ceil(B*H / 8) head groups of 8, one per XCD lane of the id.
  const int64_t tiles = ((int64_t)a.g.B * a.g.H + kXcds - 1) / kXcds * kXcds * ti * tj;
  if (tiles > 0xffffffffll) return hipErrorInvalidValue;
  if (tiles > 0) {
    if (a.g.D == 128)
      hipLaunchKernelGGL(score_kernel<128>, dim3((unsigned)tiles), dim3(256), 0, s, a, ti, tj);
    else
      hipLaunchKernelGGL(score_kernel<64>, dim3((unsigned)tiles), dim3(256), 0, s, a, ti, tj);
  }
  return hipGetLastError();
}

}  // namespace sparstar
