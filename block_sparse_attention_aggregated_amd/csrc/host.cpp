// Host layer of libsparstar: argument validation, block bookkeeping, device
// checks and kernel dispatch behind the C ABI of include/sparstar.h.
//
// Block bookkeeping follows "SparSTAR: Sparse Attention for SpaceTime
// AutoRegressive Video Synthesis", section 5 "Original-order block partition"
// (n = ceil(L / b), blocks in kernel order, not aligned to segments) and
// "Clip-Dependent Retained and Selectable Blocks" (which blocks stay dense).

#include "sparstar.h"
#include "sparstar_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

sparstar_status fail(sparstar_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sparstar_status ok() {
  g_last_error.clear();
  return SPARSTAR_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t dt) { return dt == SPARSTAR_BF16 ? 2 : 4; }

sparstar_status check_strides(const char* name, const int64_t st[3], int32_t dt) {
  const int64_t vec = 16 / elem_size(dt);  // elements per 16-byte load
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0)
      return fail(SPARSTAR_ERR_LAYOUT, "%s stride[%d] = %lld is negative", name, i, (long long)st[i]);
    if (st[i] % vec != 0)
      return fail(SPARSTAR_ERR_LAYOUT, "%s stride[%d] = %lld is not a multiple of %lld elements",
                  name, i, (long long)st[i], (long long)vec);
  }
  return SPARSTAR_OK;
}

sparstar_status check_problem_impl(const sparstar_problem* p) {
  if (!p) return fail(SPARSTAR_ERR_NULL, "problem is NULL");
  if (p->reserved != 0) return fail(SPARSTAR_ERR_SHAPE, "reserved field must be 0");
  if (p->batch < 0 || p->heads < 0)
    return fail(SPARSTAR_ERR_SHAPE, "batch (%d) and heads (%d) must be >= 0", p->batch, p->heads);
  if (p->len_q < 0 || p->len_text < 0 || p->len_ref < 0)
    return fail(SPARSTAR_ERR_SHAPE, "len_q, len_text and len_ref must be >= 0");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SPARSTAR_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", p->head_dim);
  if (p->block != 64 && p->block != 128 && p->block != 256)
    return fail(SPARSTAR_ERR_UNSUPPORTED, "block %d not built (64, 128 or 256)", p->block);
  if ((p->dtype != SPARSTAR_BF16 && p->dtype != SPARSTAR_F32) ||
      (p->out_dtype != SPARSTAR_BF16 && p->out_dtype != SPARSTAR_F32))
    return fail(SPARSTAR_ERR_UNSUPPORTED, "dtype %d / out_dtype %d not built", p->dtype, p->out_dtype);
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.0f))
    return fail(SPARSTAR_ERR_SHAPE, "softmax_scale must be finite and > 0");
  const int64_t L_k = p->len_text + p->len_ref + p->len_q;
  if (L_k > (int64_t)INT32_MAX / 2 || p->len_q > (int64_t)INT32_MAX / 2)
    return fail(SPARSTAR_ERR_SHAPE, "sequence too long (L_k = %lld)", (long long)L_k);
  const int64_t n_q = ceil_div(p->len_q, p->block), n_k = ceil_div(L_k, p->block);
  const int64_t rows = (int64_t)p->batch * p->heads * n_q;
  if (rows + 1 > (int64_t)INT32_MAX || (int64_t)p->batch * p->heads * n_k > (int64_t)INT32_MAX)
    return fail(SPARSTAR_ERR_SHAPE, "too many blocks for int32 block indexing");
  sparstar_status s;
  if ((s = check_strides("q", p->q_stride, p->dtype)) != SPARSTAR_OK) return s;
  if ((s = check_strides("k", p->k_stride, p->dtype)) != SPARSTAR_OK) return s;
  if ((s = check_strides("v", p->v_stride, p->dtype)) != SPARSTAR_OK) return s;
  if ((s = check_strides("out", p->o_stride, p->out_dtype)) != SPARSTAR_OK) return s;
  if (p->q_stride[2] < p->head_dim || p->k_stride[2] < p->head_dim ||
      p->v_stride[2] < p->head_dim || p->o_stride[2] < p->head_dim)
    return fail(SPARSTAR_ERR_LAYOUT, "token stride smaller than head_dim");
  return SPARSTAR_OK;
}

int64_t num_retained(const sparstar_problem* p, int32_t policy) {
  // The retained blocks are those that intersect [0, L_keep): the text
  // (later clips) or text + reference (clip 1).  Key blocks start at 0, so
  // this is the prefix of ceil(L_keep / b) blocks.
  const int64_t L_keep = policy == SPARSTAR_POLICY_FIRST_CLIP ? p->len_text + p->len_ref : p->len_text;
  return ceil_div(L_keep, p->block);
}

int64_t budget_impl(int64_t n, double density) {
  if (!(density > 0.0 && density <= 1.0) || n < 0) return -1;
  if (n == 0) return 0;
  int64_t k = (int64_t)std::ceil(density * (double)n - 1e-6);
  if (k < 1) k = 1;
  if (k > n) k = n;
  return k;
}

sparstar::Geometry geometry(const sparstar_problem* p) {
  sparstar::Geometry g;
  g.B = p->batch;
  g.H = p->heads;
  g.D = p->head_dim;
  g.b = p->block;
  g.L_q = p->len_q;
  g.L_k = p->len_text + p->len_ref + p->len_q;
  g.n_q = (int32_t)ceil_div(g.L_q, g.b);
  g.n_k = (int32_t)ceil_div(g.L_k, g.b);
  return g;
}

// Device check: gfx950 only.  Cached per device ordinal.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_state[kMaxDevices];  // 1 ok, 2 unsupported, 3 hip error
char g_dev_name[kMaxDevices][64];

sparstar_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPARSTAR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPARSTAR_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_dev_state[dev] = 3;
      return;
    }
    snprintf(g_dev_name[dev], sizeof g_dev_name[dev], "%s", prop.gcnArchName);
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  });
  if (g_dev_state[dev] == 3) return fail(SPARSTAR_ERR_HIP, "hipGetDeviceProperties failed on device %d", dev);
  if (g_dev_state[dev] == 2)
    return fail(SPARSTAR_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                g_dev_name[dev]);
  return SPARSTAR_OK;
}

sparstar_status launched(hipError_t e, const char* what) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(SPARSTAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

template <typename F>
sparstar_status guarded(F&& f) {
  try {
    return f();
  } catch (...) {
    return fail(SPARSTAR_ERR_HIP, "unexpected C++ exception inside libsparstar");
  }
}

sparstar_status attn_common(const sparstar_problem* p, const void* q, const void* k, const void* v,
                            void* out, sparstar::AttnArgs& a) {
  sparstar_status s = check_problem_impl(p);
  if (s != SPARSTAR_OK) return s;
  if (!q || !k || !v || !out) return fail(SPARSTAR_ERR_NULL, "q, k, v and out must be non-NULL");
  if (!is_aligned16(q) || !is_aligned16(k) || !is_aligned16(v) || !is_aligned16(out))
    return fail(SPARSTAR_ERR_LAYOUT, "q, k, v and out must be 16-byte aligned");
  a.g = geometry(p);
  a.dtype = p->dtype;
  a.out_dtype = p->out_dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.qs_b = p->q_stride[0]; a.qs_h = p->q_stride[1]; a.qs_t = p->q_stride[2];
  a.ks_b = p->k_stride[0]; a.ks_h = p->k_stride[1]; a.ks_t = p->k_stride[2];
  a.vs_b = p->v_stride[0]; a.vs_h = p->v_stride[1]; a.vs_t = p->v_stride[2];
  a.os_b = p->o_stride[0]; a.os_h = p->o_stride[1]; a.os_t = p->o_stride[2];
  a.sigma = p->softmax_scale;
  a.row_order = nullptr;
  return SPARSTAR_OK;
}

// Which attention kernel a problem runs on: the bf16 MFMA kernel takes bf16 inputs
// with D = 128 whose in-head byte offsets fit 32 bits; everything else runs the
// float32 kernel.
bool uses_mfma(const sparstar_problem* p) {
  const int64_t L_k = p->len_text + p->len_ref + p->len_q;
  const bool small_extent =
      (L_k + 256) * std::max(p->k_stride[2], p->v_stride[2]) * 2 < ((int64_t)1 << 31) &&
      (p->len_q + 256) * std::max(p->q_stride[2], p->o_stride[2]) * 4 < ((int64_t)1 << 31);
  return p->dtype == SPARSTAR_BF16 && p->head_dim == 128 && small_extent;
}

sparstar_status run_attn(const sparstar_problem* p, const sparstar::AttnArgs& a, int* counters,
                         hipStream_t st) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.n_q;
  if (rows == 0) return ok();
  sparstar_status s = check_device();
  if (s != SPARSTAR_OK) return s;
  const bool mfma = uses_mfma(p);
  return launched(mfma ? sparstar::launch_attn_mfma(a, counters, st) : sparstar::launch_attn_simt(a, st),
                  mfma ? "attention (bf16 MFMA) launch" : "attention (float32) launch");
}


// Workspace of the balanced call: the dynamic queues' counters, then the row order.
constexpr int64_t kCounterBytes = 256;
static_assert(sparstar::kAttnCounters * 4 <= kCounterBytes, "counter block too small");

int64_t balance_workspace_bytes(const sparstar_problem* p) {
  return kCounterBytes + sparstar::row_order_entries((int64_t)p->batch * p->heads,
                                                     (int32_t)ceil_div(p->len_q, p->block), p->block) *
                             (int64_t)sizeof(int32_t);
}

sparstar_status bsa_fwd_balanced_impl(const sparstar_problem* p, const void* q, const void* k, const void* v,
                                      const int32_t* row_ptr, const int32_t* col_idx, int64_t col_idx_len, void* out,
                                      float* lse, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  sparstar::AttnArgs a;
  sparstar_status s = attn_common(p, q, k, v, out, a);
  if (s != SPARSTAR_OK) return s;
  if (!row_ptr || !col_idx) return fail(SPARSTAR_ERR_NULL, "row_ptr and col_idx must be non-NULL");
  if (col_idx_len < 0) return fail(SPARSTAR_ERR_SHAPE, "col_idx_len must be >= 0");
  if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || (reinterpret_cast<uintptr_t>(col_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(workspace) & 3u))
    return fail(SPARSTAR_ERR_LAYOUT, "row_ptr, col_idx, lse and workspace must be 4-byte aligned");
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.n_q;
  const int64_t need = balance_workspace_bytes(p);
  if (workspace_bytes < need)
    return fail(SPARSTAR_ERR_CAPACITY, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)need);
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_idx_len = col_idx_len;
  if (rows == 0) return ok();
  if ((s = check_device()) != SPARSTAR_OK) return s;
  int* counters = static_cast<int*>(workspace);
  int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kCounterBytes);
  s = launched(sparstar::launch_row_order(row_ptr, (int64_t)a.g.B * a.g.H, a.g.n_q, a.g.b, col_idx_len, order,
                                          stream),
               "row order launch");
  if (s != SPARSTAR_OK) return s;
  a.row_order = order;
  return run_attn(p, a, counters, stream);
}


// Library-held scratch for sparstar_bsa_fwd_balanced_noalloc: the row-queue counters
// and the row order of the balanced call, for callers that cannot allocate.  Each
// device holds its own copy of the array until the process ends.  In host code
// `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchBytes = int64_t(1) << 20;
__device__ __align__(256) char scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

sparstar_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPARSTAR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPARSTAR_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(SPARSTAR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev]));
  *ptr = g_scratch_ptr[dev];
  return SPARSTAR_OK;
}

}  // namespace

extern "C" {

sparstar_status sparstar_check_problem(const sparstar_problem* p) {
  return guarded([&] {
    sparstar_status s = check_problem_impl(p);
    return s == SPARSTAR_OK ? ok() : s;
  });
}

int64_t sparstar_num_q_blocks(const sparstar_problem* p) {
  if (check_problem_impl(p) != SPARSTAR_OK) return -1;
  return ceil_div(p->len_q, p->block);
}

int64_t sparstar_num_k_blocks(const sparstar_problem* p) {
  if (check_problem_impl(p) != SPARSTAR_OK) return -1;
  return ceil_div(p->len_text + p->len_ref + p->len_q, p->block);
}

int64_t sparstar_num_retained(const sparstar_problem* p, int32_t policy) {
  if (check_problem_impl(p) != SPARSTAR_OK) return -1;
  if (policy != SPARSTAR_POLICY_LATER_CLIP && policy != SPARSTAR_POLICY_FIRST_CLIP) return -1;
  return num_retained(p, policy);
}

int64_t sparstar_budget(int64_t n_candidates, double density) { return budget_impl(n_candidates, density); }

int64_t sparstar_blocks_per_row(const sparstar_problem* p, double density, int32_t policy) {
  const int64_t r = sparstar_num_retained(p, policy);
  if (r < 0) return -1;
  const int64_t n_k = ceil_div(p->len_text + p->len_ref + p->len_q, p->block);
  const int64_t k = budget_impl(n_k - r, density);
  return k < 0 ? -1 : r + k;
}

int64_t sparstar_select_nnz(const sparstar_problem* p, double density, int32_t policy) {
  const int64_t per_row = sparstar_blocks_per_row(p, density, policy);
  if (per_row < 0) return -1;
  return (int64_t)p->batch * p->heads * ceil_div(p->len_q, p->block) * per_row;
}

int32_t sparstar_attention_kernel(const sparstar_problem* p) {
  if (check_problem_impl(p) != SPARSTAR_OK) return -1;
  return uses_mfma(p) ? SPARSTAR_KERNEL_MFMA_BF16 : SPARSTAR_KERNEL_F32;
}

const char* sparstar_status_string(sparstar_status s) {
  switch (s) {
    case SPARSTAR_OK: return "ok";
    case SPARSTAR_ERR_NULL: return "null pointer";
    case SPARSTAR_ERR_SHAPE: return "invalid shape";
    case SPARSTAR_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPARSTAR_ERR_LAYOUT: return "unsupported layout or alignment";
    case SPARSTAR_ERR_DENSITY: return "density out of range";
    case SPARSTAR_ERR_CAPACITY: return "output capacity too small";
    case SPARSTAR_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sparstar_last_error(void) { return g_last_error.c_str(); }

sparstar_status sparstar_pool_score(const sparstar_problem* p, const void* q, const void* k,
                                    float* q_pool, float* k_pool, float* scores, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!q || !k || !q_pool || !k_pool || !scores)
      return fail(SPARSTAR_ERR_NULL, "q, k, q_pool, k_pool and scores must be non-NULL");
    if (!is_aligned16(q) || !is_aligned16(k) || !is_aligned16(q_pool) || !is_aligned16(k_pool) ||
        !is_aligned16(scores))
      return fail(SPARSTAR_ERR_LAYOUT, "q, k, q_pool, k_pool and scores must be 16-byte aligned");
    sparstar::PoolScoreArgs a;
    a.g = geometry(p);
    if ((int64_t)a.g.B * a.g.H == 0) return ok();
    a.dtype = p->dtype;
    a.q = q;
    a.k = k;
    a.qs_b = p->q_stride[0]; a.qs_h = p->q_stride[1]; a.qs_t = p->q_stride[2];
    a.ks_b = p->k_stride[0]; a.ks_h = p->k_stride[1]; a.ks_t = p->k_stride[2];
    a.q_pool = q_pool;
    a.k_pool = k_pool;
    a.scores = scores;
    a.sigma = p->softmax_scale;
    if ((s = check_device()) != SPARSTAR_OK) return s;
    return launched(sparstar::launch_pool_score(a, (hipStream_t)stream), "pool_score launch");
  });
}

sparstar_status sparstar_select_blocks(const sparstar_problem* p, const float* scores, double density,
                                       int32_t policy, int32_t* row_ptr, int32_t* col_idx,
                                       int64_t col_idx_capacity, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!(density > 0.0 && density <= 1.0))
      return fail(SPARSTAR_ERR_DENSITY, "density %g not in (0, 1]", density);
    if (policy != SPARSTAR_POLICY_LATER_CLIP && policy != SPARSTAR_POLICY_FIRST_CLIP)
      return fail(SPARSTAR_ERR_UNSUPPORTED, "policy %d not built", policy);
    if (!scores || !row_ptr || !col_idx)
      return fail(SPARSTAR_ERR_NULL, "scores, row_ptr and col_idx must be non-NULL");
    if (!is_aligned16(scores) || (reinterpret_cast<uintptr_t>(row_ptr) & 3u) ||
        (reinterpret_cast<uintptr_t>(col_idx) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "scores must be 16-byte aligned, row_ptr/col_idx 4-byte aligned");
    const sparstar::Geometry g = geometry(p);
    const int64_t keep = std::min<int64_t>(num_retained(p, policy), g.n_k);
    const int64_t n_cand = g.n_k - keep;
    const int64_t kk = budget_impl(n_cand, density);
    const int64_t rows = (int64_t)g.B * g.H * g.n_q;
    const int64_t nnz = rows * (keep + kk);
    if (nnz > (int64_t)INT32_MAX) return fail(SPARSTAR_ERR_SHAPE, "nnz %lld exceeds int32", (long long)nnz);
    if (col_idx_capacity < nnz)
      return fail(SPARSTAR_ERR_CAPACITY, "col_idx capacity %lld < nnz %lld", (long long)col_idx_capacity,
                  (long long)nnz);
    if (n_cand > sparstar::kSelectMaxCandidates)
      return fail(SPARSTAR_ERR_UNSUPPORTED, "%lld candidate blocks per row; at most %d are built",
                  (long long)n_cand, sparstar::kSelectMaxCandidates);
    if ((s = check_device()) != SPARSTAR_OK) return s;
    sparstar::SelectArgs a;
    a.scores = scores;
    a.n_k = g.n_k;
    a.n_keep = (int32_t)keep;
    a.k = (int32_t)kk;
    a.rows = rows;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    return launched(sparstar::launch_select(a, (hipStream_t)stream), "select launch");
  });
}

sparstar_status sparstar_pool_blocks(const sparstar_problem* p, const void* q, const void* k, float* q_pool,
                                     float* k_pool, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!q || !k || !q_pool || !k_pool) return fail(SPARSTAR_ERR_NULL, "q, k, q_pool and k_pool must be non-NULL");
    if (!is_aligned16(q) || !is_aligned16(k) || !is_aligned16(q_pool) || !is_aligned16(k_pool))
      return fail(SPARSTAR_ERR_LAYOUT, "q, k, q_pool and k_pool must be 16-byte aligned");
    sparstar::PoolScoreArgs a;
    a.g = geometry(p);
    if ((int64_t)a.g.B * a.g.H == 0) return ok();
    a.dtype = p->dtype;
    a.q = q;
    a.k = k;
    a.qs_b = p->q_stride[0]; a.qs_h = p->q_stride[1]; a.qs_t = p->q_stride[2];
    a.ks_b = p->k_stride[0]; a.ks_h = p->k_stride[1]; a.ks_t = p->k_stride[2];
    a.q_pool = q_pool;
    a.k_pool = k_pool;
    a.scores = nullptr;
    a.sigma = p->softmax_scale;
    if ((s = check_device()) != SPARSTAR_OK) return s;
    return launched(sparstar::launch_pool_score(a, (hipStream_t)stream), "pool_blocks launch");
  });
}

sparstar_status sparstar_score_select(const sparstar_problem* p, const float* q_pool, const float* k_pool,
                                      double density, int32_t policy, int32_t* row_ptr, int32_t* col_idx,
                                      int64_t col_idx_capacity, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!(density > 0.0 && density <= 1.0))
      return fail(SPARSTAR_ERR_DENSITY, "density %g not in (0, 1]", density);
    if (policy != SPARSTAR_POLICY_LATER_CLIP && policy != SPARSTAR_POLICY_FIRST_CLIP)
      return fail(SPARSTAR_ERR_UNSUPPORTED, "policy %d not built", policy);
    if (!q_pool || !k_pool || !row_ptr || !col_idx)
      return fail(SPARSTAR_ERR_NULL, "q_pool, k_pool, row_ptr and col_idx must be non-NULL");
    if (!is_aligned16(q_pool) || !is_aligned16(k_pool) || (reinterpret_cast<uintptr_t>(row_ptr) & 3u) ||
        (reinterpret_cast<uintptr_t>(col_idx) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "q_pool and k_pool must be 16-byte aligned, row_ptr/col_idx 4-byte aligned");
    const sparstar::Geometry g = geometry(p);
    const int64_t keep = std::min<int64_t>(num_retained(p, policy), g.n_k);
    const int64_t n_cand = g.n_k - keep;
    const int64_t kk = budget_impl(n_cand, density);
    const int64_t rows = (int64_t)g.B * g.H * g.n_q;
    const int64_t nnz = rows * (keep + kk);
    if (nnz > (int64_t)INT32_MAX) return fail(SPARSTAR_ERR_SHAPE, "nnz %lld exceeds int32", (long long)nnz);
    if (col_idx_capacity < nnz)
      return fail(SPARSTAR_ERR_CAPACITY, "col_idx capacity %lld < nnz %lld", (long long)col_idx_capacity,
                  (long long)nnz);
    if (g.n_k > sparstar::score_select_max_keys())
      return fail(SPARSTAR_ERR_UNSUPPORTED, "%d key blocks; the fused kernel holds at most %d (use pool_score "
                  "and select_blocks)", g.n_k, sparstar::score_select_max_keys());
    if ((s = check_device()) != SPARSTAR_OK) return s;
    sparstar::ScoreSelectArgs a;
    a.g = g;
    a.q_pool = q_pool;
    a.k_pool = k_pool;
    a.sigma = p->softmax_scale;
    a.n_keep = (int32_t)keep;
    a.k = (int32_t)kk;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    return launched(sparstar::launch_score_select(a, (hipStream_t)stream), "score_select launch");
  });
}

int64_t sparstar_bsa_workspace_bytes(const sparstar_problem* p) {
  if (check_problem_impl(p) != SPARSTAR_OK) return -1;
  return kCounterBytes;
}

sparstar_status sparstar_bsa_fwd(const sparstar_problem* p, const void* q, const void* k, const void* v,
                                 const int32_t* row_ptr, const int32_t* col_idx, int64_t col_idx_len,
                                 void* out, float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar::AttnArgs a;
    sparstar_status s = attn_common(p, q, k, v, out, a);
    if (s != SPARSTAR_OK) return s;
    if (!row_ptr || !col_idx) return fail(SPARSTAR_ERR_NULL, "row_ptr and col_idx must be non-NULL");
    if (col_idx_len < 0) return fail(SPARSTAR_ERR_SHAPE, "col_idx_len must be >= 0");
    if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || (reinterpret_cast<uintptr_t>(col_idx) & 3u) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(workspace) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "row_ptr, col_idx, lse and workspace must be 4-byte aligned");
    if (workspace && workspace_bytes < kCounterBytes)
      return fail(SPARSTAR_ERR_CAPACITY, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                  (long long)kCounterBytes);
    a.lse = lse;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.col_idx_len = col_idx_len;
    return run_attn(p, a, static_cast<int*>(workspace), (hipStream_t)stream);
  });
}

sparstar_status dense_attn_fwd(const sparstar_problem* p, const void* q, const void* k, const void* v,
                               void* out, float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar::AttnArgs a;
    sparstar_status s = attn_common(p, q, k, v, out, a);
    if (s != SPARSTAR_OK) return s;
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(workspace) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "lse and workspace must be 4-byte aligned");
    if (workspace && workspace_bytes < kCounterBytes)
      return fail(SPARSTAR_ERR_CAPACITY, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                  (long long)kCounterBytes);
    a.lse = lse;
    a.row_ptr = nullptr;
    a.col_idx = nullptr;
    a.col_idx_len = 0;
    return run_attn(p, a, static_cast<int*>(workspace), (hipStream_t)stream);
  });
}

sparstar_status sparstar_block_mass(const sparstar_problem* p, const void* q, const void* k, const float* lse,
                                    float* mass, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!q || !k || !lse || !mass) return fail(SPARSTAR_ERR_NULL, "q, k, lse and mass must be non-NULL");
    if (!is_aligned16(q) || !is_aligned16(k) || (reinterpret_cast<uintptr_t>(lse) & 3u) ||
        (reinterpret_cast<uintptr_t>(mass) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "q and k must be 16-byte aligned, lse and mass 4-byte aligned");
    sparstar::MassArgs a;
    a.g = geometry(p);
    if ((int64_t)a.g.B * a.g.H * a.g.n_q == 0 || a.g.n_k == 0) return ok();
    a.dtype = p->dtype;
    a.q = q;
    a.k = k;
    a.qs_b = p->q_stride[0]; a.qs_h = p->q_stride[1]; a.qs_t = p->q_stride[2];
    a.ks_b = p->k_stride[0]; a.ks_h = p->k_stride[1]; a.ks_t = p->k_stride[2];
    a.lse = lse;
    a.mass = mass;
    a.sigma = p->softmax_scale;
    a.small_extent = (a.g.L_k + 256) * a.ks_t * 2 < ((int64_t)1 << 31);
    if ((s = check_device()) != SPARSTAR_OK) return s;
    return launched(sparstar::launch_block_mass(a, (hipStream_t)stream), "block_mass launch");
  });
}

sparstar_status sparstar_selection_mass(const sparstar_problem* p, const float* mass, const int32_t* row_ptr,
                                        const int32_t* col_idx, int64_t col_idx_len, float* row_mass,
                                        void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!mass || !row_ptr || !col_idx || !row_mass)
      return fail(SPARSTAR_ERR_NULL, "mass, row_ptr, col_idx and row_mass must be non-NULL");
    if (col_idx_len < 0) return fail(SPARSTAR_ERR_SHAPE, "col_idx_len must be >= 0");
    if ((reinterpret_cast<uintptr_t>(mass) & 3u) || (reinterpret_cast<uintptr_t>(row_ptr) & 3u) ||
        (reinterpret_cast<uintptr_t>(col_idx) & 3u) || (reinterpret_cast<uintptr_t>(row_mass) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "mass, row_ptr, col_idx and row_mass must be 4-byte aligned");
    const sparstar::Geometry g = geometry(p);
    sparstar::SelMassArgs a;
    a.mass = mass;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.col_idx_len = col_idx_len;
    a.rows = (int64_t)g.B * g.H * g.n_q;
    a.n_q = g.n_q;
    a.n_k = g.n_k;
    a.b = g.b;
    a.L_q = g.L_q;
    a.out = row_mass;
    if (a.rows == 0) return ok();
    if ((s = check_device()) != SPARSTAR_OK) return s;
    return launched(sparstar::launch_selection_mass(a, (hipStream_t)stream), "selection_mass launch");
  });
}

sparstar_status sparstar_window_scores(const sparstar_problem* p, float* scores, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (!scores) return fail(SPARSTAR_ERR_NULL, "scores must be non-NULL");
    if (!is_aligned16(scores)) return fail(SPARSTAR_ERR_LAYOUT, "scores must be 16-byte aligned");
    const sparstar::Geometry g = geometry(p);
    const int64_t bh = (int64_t)g.B * g.H;
    if (bh * g.n_q * g.n_k == 0) return ok();
    if ((s = check_device()) != SPARSTAR_OK) return s;
    return launched(sparstar::launch_window_scores(scores, bh, g.n_q, g.n_k, g.b, p->len_text + p->len_ref,
                                                   (hipStream_t)stream),
                    "window_scores launch");
  });
}

sparstar_status sparstar_token_topk_mass(const sparstar_problem* p, const void* q, const void* k, const float* lse,
                                         const int64_t* rows, int64_t n_rows, int64_t keep_tokens,
                                         int64_t k_tokens, float* out, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    if (n_rows < 0 || keep_tokens < 0 || k_tokens < 0)
      return fail(SPARSTAR_ERR_SHAPE, "n_rows, keep_tokens and k_tokens must be >= 0");
    if (n_rows == 0) return ok();
    if (!q || !k || !lse || !rows || !out) return fail(SPARSTAR_ERR_NULL, "q, k, lse, rows and out must be non-NULL");
    if (!is_aligned16(q) || !is_aligned16(k) || (reinterpret_cast<uintptr_t>(lse) & 3u) ||
        (reinterpret_cast<uintptr_t>(rows) & 7u) || (reinterpret_cast<uintptr_t>(out) & 3u))
      return fail(SPARSTAR_ERR_LAYOUT, "q, k 16-byte, rows 8-byte, lse and out 4-byte aligned");
    sparstar::TopkArgs a;
    a.g = geometry(p);
    if ((int64_t)a.g.B * a.g.H * a.g.L_q == 0) return fail(SPARSTAR_ERR_SHAPE, "no queries to list");
    a.dtype = p->dtype;
    a.q = q;
    a.k = k;
    a.qs_b = p->q_stride[0]; a.qs_h = p->q_stride[1]; a.qs_t = p->q_stride[2];
    a.ks_b = p->k_stride[0]; a.ks_h = p->k_stride[1]; a.ks_t = p->k_stride[2];
    a.lse = lse;
    a.rows = rows;
    a.n_rows = n_rows;
    a.keep_tokens = keep_tokens;
    a.k_tokens = k_tokens;
    a.sigma = p->softmax_scale;
    a.out = out;
    if ((s = check_device()) != SPARSTAR_OK) return s;
    return launched(sparstar::launch_token_topk(a, (hipStream_t)stream), "token_topk_mass launch");
  });
}

int64_t sparstar_balance_workspace_bytes(const sparstar_problem* p) {
  if (check_problem_impl(p) != SPARSTAR_OK) return -1;
  return balance_workspace_bytes(p);
}

sparstar_status sparstar_bsa_fwd_balanced(const sparstar_problem* p, const void* q, const void* k, const void* v,
                                          const int32_t* row_ptr, const int32_t* col_idx, int64_t col_idx_len,
                                          void* out, float* lse, void* workspace, int64_t workspace_bytes,
                                          void* stream) {
  return guarded([&]() -> sparstar_status {
    if (!workspace) return fail(SPARSTAR_ERR_NULL, "workspace must be non-NULL");
    return bsa_fwd_balanced_impl(p, q, k, v, row_ptr, col_idx, col_idx_len, out, lse, workspace, workspace_bytes,
                                 (hipStream_t)stream);
  });
}

sparstar_status sparstar_bsa_fwd_balanced_noalloc(const sparstar_problem* p, const void* q, const void* k,
                                                  const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                                                  int64_t col_idx_len, void* out, float* lse, void* stream) {
  return guarded([&]() -> sparstar_status {
    sparstar_status s = check_problem_impl(p);
    if (s != SPARSTAR_OK) return s;
    const int64_t need = balance_workspace_bytes(p);
    if (need > kScratchBytes)
      return fail(SPARSTAR_ERR_CAPACITY,
                  "the problem needs %lld bytes of row queue and order; the library's scratch holds %lld "
                  "(use sparstar_bsa_fwd_balanced with a workspace)",
                  (long long)need, (long long)kScratchBytes);
    void* ws = nullptr;
    if ((int64_t)p->batch * p->heads * ceil_div(p->len_q, p->block) > 0) {
      if ((s = check_device()) != SPARSTAR_OK) return s;
      if ((s = scratch_on_current_device(&ws)) != SPARSTAR_OK) return s;
    }
    return bsa_fwd_balanced_impl(p, q, k, v, row_ptr, col_idx, col_idx_len, out, lse, ws, kScratchBytes,
                                 (hipStream_t)stream);
  });
}

int64_t sparstar_mfma_probe_sink_len(void) {
  const int64_t wgs = sparstar::mfma_probe_workgroups();
  return wgs > 0 ? wgs * 256 : -1;
}

sparstar_status sparstar_mfma_probe(int32_t rounds, float* sink, int64_t sink_len, double* flops, void* stream) {
  return guarded([&]() -> sparstar_status {
    if (rounds < 1) return fail(SPARSTAR_ERR_SHAPE, "rounds must be >= 1, got %d", rounds);
    if (!sink) return fail(SPARSTAR_ERR_NULL, "sink must be non-NULL");
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return fail(SPARSTAR_ERR_LAYOUT, "sink must be 4-byte aligned");
    sparstar_status s = check_device();
    if (s != SPARSTAR_OK) return s;
    const int64_t wgs = sparstar::mfma_probe_workgroups();
    if (wgs <= 0) return fail(SPARSTAR_ERR_HIP, "could not query the CU count");
    if (sink_len < wgs * 256)
      return fail(SPARSTAR_ERR_CAPACITY, "sink of %lld floats, %lld needed", (long long)sink_len,
                  (long long)(wgs * 256));
    if ((s = launched(sparstar::launch_mfma_probe(rounds, sink, wgs, (hipStream_t)stream), "mfma_probe launch")) !=
        SPARSTAR_OK)
      return s;
    if (flops) *flops = sparstar::mfma_probe_flops(rounds, wgs);
    return ok();
  });
}

}  // extern "C"
