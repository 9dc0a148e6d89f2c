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

namespace sparstar {
namespace {

constexpr int kWaves = 4;

// Larger float -> larger unsigned key; -0.0 is folded onto +0.0 first.
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  return __popcll(mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

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

  // Retained prefix.
  for (int j = lane; j < a.n_keep; j += 64) out[j] = j;
  if (a.k == 0) return;

  // Radix select of the k-th largest key among the valid candidates.
  uint32_t prefix = 0, pmask = 0;
  int remaining = a.k;  // rank still to find inside the current prefix bucket
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = lane; i < 256; i += 64) hist[i] = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int c = lane + 64 * t;
      if (c < n_cand && (key[t] & pmask) == prefix) atomicAdd(&hist[(key[t] >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // Lane l owns bins 4l .. 4l+3.  Suffix sums from the top bin downwards.
    const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
    const uint32_t mine = h0 + h1 + h2 + h3;
    // Inclusive suffix scan of the per-lane totals over lanes l .. 63, then
    // minus the lane's own total: the count in all bins above this lane's.
    uint32_t acc = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_down(acc, off);
      if (lane + off < 64) acc += v;
    }
    const uint32_t above = acc - mine;
    // Find the bin d (descending) where the cumulative count from the top reaches 'remaining'.
    const uint32_t c3 = above + h3, c2 = c3 + h2, c1 = c2 + h1, c0 = c1 + h0;
    const uint32_t rem = (uint32_t)remaining;
    int digit = -1;
    uint32_t before = 0;
    if (above < rem && c3 >= rem) { digit = 4 * lane + 3; before = above; }
    else if (c3 < rem && c2 >= rem) { digit = 4 * lane + 2; before = c3; }
    else if (c2 < rem && c1 >= rem) { digit = 4 * lane + 1; before = c2; }
    else if (c1 < rem && c0 >= rem) { digit = 4 * lane + 0; before = c1; }
    const uint64_t who = __ballot(digit >= 0);
    const int src = __ffsll((unsigned long long)who) - 1;
    const int d_sel = __shfl(digit, src);
    const uint32_t b_sel = __shfl(before, src);
    prefix |= (uint32_t)d_sel << shift;
    pmask |= 255u << shift;
    remaining -= (int)b_sel;
    __builtin_amdgcn_wave_barrier();
  }
  // prefix is the exact key of the k-th best candidate; 'remaining' of the
  // candidates equal to it are taken (the lowest block indices first).
  const uint32_t thr = prefix;
  int eq_seen = 0, taken = 0;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int c = lane + 64 * t;
    const bool valid = c < n_cand;
    const bool gt = valid && key[t] > thr;
    const bool eq = valid && key[t] == thr;
    const uint64_t eq_mask = __ballot(eq);
    const int eq_rank = eq_seen + lanes_below(eq_mask);
    const bool take = gt || (eq && eq_rank < remaining);
    const uint64_t take_mask = __ballot(take);
    if (take) out[a.n_keep + taken + lanes_below(take_mask)] = a.n_keep + c;
    eq_seen += __popcll(eq_mask);
    taken += __popcll(take_mask);
  }
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

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int64_t n = a.rows + 1;
  hipLaunchKernelGGL(row_ptr_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.row_ptr, a.rows,
                     a.n_keep + a.k);
  if (a.rows == 0) return hipGetLastError();
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
