// Internal interface between the host layer (host.cpp) and the kernel files.
// Everything here has been validated by the host layer before a launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparstar {

// Geometry of one scale, already derived on the host.
struct Geometry {
  int32_t B, H, D, b;
  int64_t L_q, L_k;
  int32_t n_q, n_k;
};

struct PoolScoreArgs {
  Geometry g;
  int dtype;                 // 0 bf16, 1 f32
  const void* q;
  const void* k;
  int64_t qs_b, qs_h, qs_t;  // element strides
  int64_t ks_b, ks_h, ks_t;
  float* q_pool;             // [B,H,n_q,D]
  float* k_pool;             // [B,H,n_k,D]
  float* scores;             // [B,H,n_q,n_k]; nullptr: pooling only
  float sigma;
};

// Scores and selection in one kernel (no score matrix in memory).
struct ScoreSelectArgs {
  Geometry g;
  const float* q_pool;       // [B,H,n_q,D] contiguous
  const float* k_pool;       // [B,H,n_k,D] contiguous
  float sigma;
  int32_t n_keep;            // retained prefix [0, n_keep)
  int32_t k;                 // candidates taken per row
  int32_t* row_ptr;          // [B*H*n_q + 1]
  int32_t* col_idx;
};

struct SelectArgs {
  const float* scores;       // [rows, n_k]
  int32_t n_k;
  int32_t n_keep;            // retained prefix [0, n_keep)
  int32_t k;                 // candidates taken per row
  int64_t rows;              // B*H*n_q
  int32_t* row_ptr;          // [rows + 1]
  int32_t* col_idx;
};

struct AttnArgs {
  Geometry g;
  int dtype;                 // q/k/v dtype
  int out_dtype;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;                // nullable, [B,H,L_q]
  int64_t qs_b, qs_h, qs_t;
  int64_t ks_b, ks_h, ks_t;
  int64_t vs_b, vs_h, vs_t;
  int64_t os_b, os_h, os_t;
  const int32_t* row_ptr;    // nullptr => dense (every key block)
  const int32_t* col_idx;
  int64_t col_idx_len;
  float sigma;
  const int32_t* row_order;  // nullable: per (head, XCD) segment, the query blocks longest list first
};

// Retained attention mass (dense softmax mass per block pair, of a selection,
// and the token-wise Top-K bound).
struct MassArgs {
  Geometry g;
  int dtype;
  const void* q;
  const void* k;
  int64_t qs_b, qs_h, qs_t;
  int64_t ks_b, ks_h, ks_t;
  const float* lse;          // [B,H,L_q] packed, natural-log sum-exp of sigma*q.k over all keys
  float* mass;               // [B,H,n_q,n_k]
  float sigma;
  bool small_extent;         // in-head byte offsets of K below 2^31 (MFMA path)
};

struct SelMassArgs {
  const float* mass;         // [rows, n_k]
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t col_idx_len;
  int64_t rows;              // B*H*n_q
  int32_t n_q, n_k, b;
  int64_t L_q;
  float* out;                // [rows]
};

struct TopkArgs {
  Geometry g;
  int dtype;
  const void* q;
  const void* k;
  int64_t qs_b, qs_h, qs_t;
  int64_t ks_b, ks_h, ks_t;
  const float* lse;          // [B,H,L_q] packed
  const int64_t* rows;       // [n_rows]: query index bh*L_q + t
  int64_t n_rows;
  int64_t keep_tokens, k_tokens;
  float sigma;
  float* out;                // [n_rows]
};

hipError_t launch_pool_score(const PoolScoreArgs& a, hipStream_t s);
hipError_t launch_block_mass(const MassArgs& a, hipStream_t s);
hipError_t launch_selection_mass(const SelMassArgs& a, hipStream_t s);
hipError_t launch_window_scores(float* out, int64_t bh, int n_q, int n_k, int b, int64_t offset, hipStream_t s);
hipError_t launch_token_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
// row_ptr[r] = r * per_row for r = 0 .. rows.
hipError_t launch_row_ptr(int32_t* row_ptr, int64_t rows, int32_t per_row, hipStream_t s);
// Largest n_k the fused score-and-select kernel holds (a strip's keys in LDS).
int score_select_max_keys();
hipError_t launch_score_select(const ScoreSelectArgs& a, hipStream_t s);

// Matrix-core rate probe (measurement helper): workgroups per launch on the current
// device (-1 on error), the launch, and the multiply-add flops of one launch.
int64_t mfma_probe_workgroups();
hipError_t launch_mfma_probe(int32_t rounds, float* sink, int64_t workgroups, hipStream_t s);
double mfma_probe_flops(int32_t rounds, int64_t workgroups);
// Attention row mapping: the query blocks of a head are split into S contiguous
// segments of per = ceil(n_q / S) blocks; workgroup id w runs on XCD
// x = w % kXcds, which takes segment x % S of head (w / kXcds / per) * (kXcds / S)
// + x / S, so kXcds / S heads are in flight at a time, each on S XCDs.  S = 4 at
// b = 128 and 256 when the number of heads B*H is even, else 8 (measured: four is
// faster at b = 128 and 256, eight at b = 64; with an odd head count the last head
// would leave half the XCDs idle).
constexpr int kXcds = 8;
constexpr int segments_per_head(int b, int64_t bh) { return (b != 64 && bh % 2 == 0) ? 4 : 8; }
// Query blocks of each (head, segment) ordered by list length, longest first:
// order[(bh * S + x) * ceil(n_q / S) + m], -1 past a segment's end.
int64_t row_order_entries(int64_t bh, int32_t n_q, int32_t b);
hipError_t launch_row_order(const int32_t* row_ptr, int64_t bh, int32_t n_q, int32_t b, int64_t col_idx_len,
                            int32_t* order, hipStream_t s);
// bf16 inputs, D = 128, b = 64, 128 or 256, in-head K/V byte offsets below 2^31 (MFMA path).
// A persistent grid: with counters (kAttnCounters ints, zeroed by the launch itself) the
// row queues are dynamic (atomic pops, idle workgroups take other XCDs' rows); without,
// each workgroup runs a fixed share of its XCD's queue.
constexpr int kAttnCounters = kXcds;
hipError_t launch_attn_mfma(const AttnArgs& a, int* counters, hipStream_t s);
// Any supported shape/dtype (float32 path).
hipError_t launch_attn_simt(const AttnArgs& a, hipStream_t s);

// Largest candidate count one select wavefront holds in registers.
constexpr int kSelectMaxCandidates = 64 * 64;

}  // namespace sparstar
