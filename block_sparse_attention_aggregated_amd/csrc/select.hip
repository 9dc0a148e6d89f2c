// Clip-aware per-row top-k block selection, written as CSR.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Clip-Dependent Retained and Selectable Blocks" and appendix A.7
// "Later-clip schedule": the designated context blocks stay dense (the prefix
// [0, n_keep) of key blocks), the remaining blocks of the row are ranked by
// score and the best k kept; section 5 "Forward-Only Sparse Execution": only
// the forward fields (per query block, the count and the indices of its
// visible key blocks) are produced.  Equal scores go to the lower block index.
//
// One wavefront per row.  Each lane holds up to T candidate keys in
// registers (candidate c = lane + 64 * t), as order-preserving uint32 images
// of the float32 scores.  A 4-pass MSB-first radix select (8 bits per pass,
// 256-bin LDS histogram per wavefront) finds the exact key of the k-th best
// candidate and how many candidates equal to it are taken; a final pass in
// ascending block order emits the retained prefix and the taken candidates
// with wave ballots, so the output is ascending without any sort.

#include "sparstar_internal.h"
#include "select_row.h"

namespace sparstar {
namespace {

constexpr int kWaves = 4;

using select_detail::order_key;

template <int T>
__global__ __launch_bounds__(64 * kWaves) void select_kernel(SelectArgs a) {
  __shared__ uint32_t hist_all[kWaves][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (row >= a.rows) return;  // whole wavefront leaves together; no block-level barrier below
  uint32_t* hist = hist_all[wave];

  const float* srow = a.scores + row * a.n_k;
  const int n_cand = a.n_k - a.n_keep;
  const int per_row = a.n_keep + a.k;
  int32_t* out = a.col_idx + row * (int64_t)per_row;

  uint32_t key[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int c = lane + 64 * t;
    key[t] = (c < n_cand) ? order_key(srow[a.n_keep + c]) : 0u;
  }

  sparstar::select_detail::select_row<T>(key, n_cand, a.n_keep, a.k, out, hist);
}

__global__ void row_ptr_kernel(int32_t* row_ptr, int64_t rows, int32_t per_row) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r <= rows) row_ptr[r] = (int32_t)(r * per_row);
}

template <int T>
void launch_t(const SelectArgs& a, hipStream_t s) {
  const int64_t wgs = (a.rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(select_kernel<T>, dim3((unsigned)wgs), dim3(64 * kWaves), 0, s, a);
}

}  // namespace

hipError_t launch_row_ptr(int32_t* row_ptr, int64_t rows, int32_t per_row, hipStream_t s) {
  const int64_t n = rows + 1;
  hipLaunchKernelGGL(row_ptr_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, row_ptr, rows, per_row);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  hipError_t e = launch_row_ptr(a.row_ptr, a.rows, a.n_keep + a.k, s);
  if (e != hipSuccess || a.rows == 0) return e;
  const int n_cand = a.n_k - a.n_keep;
  if (n_cand <= 64 * 4) launch_t<4>(a, s);
  else if (n_cand <= 64 * 8) launch_t<8>(a, s);
  else if (n_cand <= 64 * 16) launch_t<16>(a, s);
  else if (n_cand <= 64 * 24) launch_t<24>(a, s);
  else if (n_cand <= 64 * 32) launch_t<32>(a, s);
  else if (n_cand <= 64 * 40) launch_t<40>(a, s);
  else if (n_cand <= 64 * 48) launch_t<48>(a, s);
  else if (n_cand <= 64 * 64) launch_t<64>(a, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sparstar
