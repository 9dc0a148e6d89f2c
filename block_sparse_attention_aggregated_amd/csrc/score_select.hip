// Aggregated-QK block scores and clip-aware top-k selection in one kernel, with
// no score matrix in memory.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Per-head aggregated query-key score" (one score per query block,
// key block and head, here sigma * <qbar_i, kbar_j>) and "Clip-Dependent
// Retained and Selectable Blocks" (the retained prefix plus the k best
// candidates of each row).
//
// One workgroup of 16 wavefronts per (batch * head, strip of 32 query blocks):
//   1. the strip's scores against every key block, 32 x 32 tiles on the float32
//      matrix cores (v_mfma_f32_32x32x2_f32), written to LDS as order-preserving
//      uint32 keys [32][n_k]; wavefront w computes key tiles w, w + 16, ...;
//   2. wavefront w ranks the strip's rows w and w + 16 from LDS with the shared
//      row selector.
// The strip's keys fill nearly all of the LDS, so one workgroup runs per CU; 16
// wavefronts (four per SIMD, 110 VGPRs each) hide more of the latency of the
// pooled-row loads and of the selector's LDS atomics than 8 (0.20 against
// 0.23 ms at 720p).
// Each tile runs the score kernel's MFMA sequence: for feature chunk c (32
// features), step q (4 features) and element e, lane l supplies feature
// 32 c + 16 (l >> 5) + 4 q + e of query row l & 31 and of key row l & 31, and
// the result is scaled by sigma after the last step; the scores, and so the
// block lists, are the same bit for bit as from the score and selection
// kernels.  The keys of a strip take 32 * n_k * 4 bytes of LDS: n_k is at most
// kMaxKeys.

#include "sparstar_internal.h"
#include "select_row.h"

namespace sparstar {
namespace {

constexpr int kFWaves = 16;
constexpr int kStrip = 32;
constexpr int kHistWords = kFWaves * 256;
constexpr int kKeyWords = (160 * 1024 - kHistWords * 4) / 4;  // LDS words left for keys

template <int D, int T>
__global__ __launch_bounds__(64 * kFWaves, 2) void score_select_kernel(ScoreSelectArgs a, int strips) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int kChunks = D / 32;
  __shared__ uint32_t keys[kKeyWords];
  __shared__ uint32_t hist_all[kHistWords];

  const Geometry& g = a.g;
  const int64_t bh = blockIdx.x / strips;
  const int strip = (int)(blockIdx.x - bh * strips);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r32 = lane & 31, hl = lane >> 5;
  const int n_k = g.n_k, q0 = strip * kStrip;
  const float* qp = a.q_pool + bh * (int64_t)g.n_q * D;
  const float* kp = a.k_pool + bh * (int64_t)n_k * D;

  // 1. Scores.  Query rows past n_q repeat the last row; their keys are not stored.
  f32x4 af[kChunks][4];
  {
    const float* qrow = qp + (int64_t)min(q0 + r32, g.n_q - 1) * D + 16 * hl;
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) af[c][q] = *reinterpret_cast<const f32x4*>(qrow + 32 * c + 4 * q);
  }
  const int n_tiles = (n_k + 31) / 32;
  for (int jt = wave; jt < n_tiles; jt += kFWaves) {
    const float* krow = kp + (int64_t)min(jt * 32 + r32, n_k - 1) * D + 16 * hl;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      f32x4 bf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bf[q] = *reinterpret_cast<const f32x4*>(krow + 32 * c + 4 * q);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[c][q][e], bf[q][e], acc, 0, 0, 0);
    }
    // Register r of a lane holds query row 8 (r >> 2) + 4 hl + (r & 3), key column r32.
    const int j = jt * 32 + r32;
    if (j < n_k) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * hl + (r & 3);
        if (q0 + i < g.n_q) keys[i * n_k + j] = select_detail::order_key(a.sigma * acc[r]);
      }
    }
  }
  __syncthreads();

  // 2. Selection of the strip's rows.
  const int n_cand = n_k - a.n_keep;
  const int per_row = a.n_keep + a.k;
  for (int i = wave; i < kStrip; i += kFWaves) {
    if (q0 + i >= g.n_q) break;  // uniform over the wavefront
    const uint32_t* krow = keys + i * n_k + a.n_keep;
    uint32_t key[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int c = lane + 64 * t;
      key[t] = c < n_cand ? krow[c] : 0u;
    }
    int32_t* out = a.col_idx + (bh * (int64_t)g.n_q + q0 + i) * per_row;
    select_detail::select_row<T>(key, n_cand, a.n_keep, a.k, out, hist_all + wave * 256);
  }
}

template <int D, int T>
void launch_dt(const ScoreSelectArgs& a, int strips, int64_t wgs, hipStream_t s) {
  hipLaunchKernelGGL((score_select_kernel<D, T>), dim3((unsigned)wgs), dim3(64 * kFWaves), 0, s, a, strips);
}

template <int D>
hipError_t launch_d(const ScoreSelectArgs& a, int strips, int64_t wgs, hipStream_t s) {
  const int n_cand = a.g.n_k - a.n_keep;
  if (n_cand <= 64 * 4) launch_dt<D, 4>(a, strips, wgs, s);
  else if (n_cand <= 64 * 8) launch_dt<D, 8>(a, strips, wgs, s);
  else if (n_cand <= 64 * 16) launch_dt<D, 16>(a, strips, wgs, s);
  else if (n_cand <= 64 * 24) launch_dt<D, 24>(a, strips, wgs, s);
  else return hipErrorInvalidValue;
  return hipSuccess;
}

}  // namespace

int score_select_max_keys() { return kKeyWords / kStrip; }

hipError_t launch_score_select(const ScoreSelectArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.n_q;
  hipError_t e = launch_row_ptr(a.row_ptr, rows, a.n_keep + a.k, s);
  if (e != hipSuccess || rows == 0 || a.k + a.n_keep == 0) return e;
  if (a.g.n_k > score_select_max_keys() || a.g.n_k - a.n_keep > 64 * 24) return hipErrorInvalidValue;
  const int strips = (a.g.n_q + kStrip - 1) / kStrip;
  const int64_t wgs = (int64_t)a.g.B * a.g.H * strips;
  if (wgs > 0xffffffffll) return hipErrorInvalidValue;
  e = a.g.D == 128 ? launch_d<128>(a, strips, wgs, s) : launch_d<64>(a, strips, wgs, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace sparstar
