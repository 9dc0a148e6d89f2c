// One row of the clip-aware top-k block selection, ranked by one wavefront.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 5 "Clip-Dependent Retained and Selectable Blocks": the retained prefix
// [0, n_keep) of key blocks, then the k best candidates by score, equal scores to
// the lower block index, in ascending order.
//
// The wavefront holds the candidates' order-preserving uint32 images in
// registers (candidate c = lane + 64 t in key[t]; 0 for c >= n_cand).  A 4-pass
// MSB-first radix select (8 bits per pass, a 256-bin LDS histogram per
// wavefront) finds the exact key of the k-th best candidate and how many
// candidates equal to it are taken; a last pass in ascending block order writes
// the taken candidates with wave ballots, so the row comes out sorted without a
// sort.  Shared by the selection kernel (keys from the scores in memory) and the
// fused score-and-select kernel (keys from scores it computes into LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparstar {
namespace select_detail {

// Larger float -> larger unsigned key; -0.0 is folded onto +0.0 first.
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  return __popcll(mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

// out: the row's n_keep + k entries; hist: this wavefront's 256 LDS words.
template <int T>
__device__ inline void select_row(const uint32_t (&key)[T], int n_cand, int n_keep, int k, int32_t* out,
                                  uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  // Retained prefix.
  for (int j = lane; j < n_keep; j += 64) out[j] = j;
  if (k == 0) return;

  // Radix select of the k-th largest key among the valid candidates.
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;  // rank still to find inside the current prefix bucket
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
    if (take) out[n_keep + taken + lanes_below(take_mask)] = n_keep + c;
    eq_seen += __popcll(eq_mask);
    taken += __popcll(take_mask);
  }
}

}  // namespace select_detail
}  // namespace sparstar
