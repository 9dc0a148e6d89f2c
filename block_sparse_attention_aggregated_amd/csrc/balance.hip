// Row order for uneven block lists: longest list first, within each segment of a head.
//
// The block-sparse attention forward ("SparSTAR: Sparse Attention for
// SpaceTime AutoRegressive Video Synthesis", section 5 "Forward-Only Sparse
// Execution") runs one workgroup per query-block row.  Its workgroups are
// numbered so that a head's query blocks form S contiguous segments
// [x * per, (x + 1) * per) (per = ceil(n_q / S), S = segments_per_head(b, B*H)), each
// run by one XCD, heads in order: the rows in flight belong to one or two heads,
// whose K and V stay in the Infinity Cache.  With uneven lists the rows handed
// out last set the tail: a long row started last keeps part of the GPU busy
// alone.  This kernel reorders the rows of each segment by list length, longest
// first (the longest-processing-time order), and keeps the order of heads and
// segments.  The sort is stable, so lists of equal length keep the plain order
// exactly.
//
// One workgroup per segment; each row's rank is the number of rows of the
// segment with a longer list, or an equally long one and a lower index.
// order[(bh * S + x) * per + m] is the query block of the m-th row of segment
// (bh, x), or -1 past the segment's end.

#include "sparstar_internal.h"

namespace sparstar {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void row_order_kernel(const int32_t* row_ptr, int32_t n_q, int32_t per,
                                                             int32_t segs_per_head, int64_t col_idx_len,
                                                             int32_t* order) {
  extern __shared__ int32_t len[];  // [per]
  const int64_t seg = blockIdx.x;   // bh * segs_per_head + x
  const int64_t bh = seg / segs_per_head;
  const int x = (int)(seg - bh * segs_per_head);
  const int q0 = x * per;
  const int n = max(0, min(per, n_q - q0));
  for (int m = threadIdx.x; m < n; m += kThreads) {
    const int64_t r = bh * n_q + q0 + m;
    int64_t beg = row_ptr[r], end = row_ptr[r + 1];
    if (beg < 0) beg = 0;
    if (end > col_idx_len) end = col_idx_len;
    const int64_t l = end > beg ? end - beg : 0;
    len[m] = (int32_t)(l < 0x7fffffff ? l : 0x7fffffff);
  }
  __syncthreads();
  int32_t* out = order + seg * per;
  for (int m = threadIdx.x; m < per; m += kThreads) {
    if (m >= n) {
      out[m] = -1;
      continue;
    }
    const int32_t lm = len[m];
    int rank = 0;
    for (int u = 0; u < n; ++u) rank += (len[u] > lm) | (len[u] == lm && u < m);
    out[rank] = q0 + m;
  }
}

}  // namespace

int64_t row_order_entries(int64_t bh, int32_t n_q, int32_t b) {
  const int S = segments_per_head(b, bh);
  return bh * S * (int64_t)((n_q + S - 1) / S);
}

hipError_t launch_row_order(const int32_t* row_ptr, int64_t bh, int32_t n_q, int32_t b, int64_t col_idx_len,
                            int32_t* order, hipStream_t s) {
  if (bh == 0 || n_q == 0) return hipSuccess;
  const int32_t S = segments_per_head(b, bh);
  const int32_t per = (n_q + S - 1) / S;
  const int64_t segs = bh * S;
  if (segs > 0xffffffffll || (size_t)per * sizeof(int32_t) > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_order_kernel, dim3((unsigned)segs), dim3(kThreads), (size_t)per * sizeof(int32_t), s,
                     row_ptr, n_q, per, S, col_idx_len, order);
  return hipGetLastError();
}

}  // namespace sparstar
