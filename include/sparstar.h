/*
 * sparstar.h -- C ABI of libsparstar: SparSTAR dynamic block-sparse attention
 * for one expensive scale of spacetime-autoregressive video generation, on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video
 * Synthesis" (full text), section 5 "Method".  For every (batch, head):
 *   1. mean-pool contiguous query and key blocks of b tokens        (sparstar_pool_score)
 *   2. score every (query block, key block) pair, S = sigma*Qbar*Kbar^T (sparstar_pool_score)
 *   3. keep the designated context blocks, rank the rest per query
 *      block and keep the top fraction rho, as a CSR block list     (sparstar_select_blocks)
 *   4. attend each query block to its listed key blocks only       (sparstar_bsa_fwd)
 * and a dense forward over every key block as the density-1 baseline
 * (dense_attn_fwd).
 *
 * Layout.  Q is [B, H, L_q, D]; K and V are [B, H, L_k, D] with the key
 * sequence ordered [text | reference | current], L_k = L_text + L_ref + L_q:
 * the current-scale tokens are both the queries and the last L_q keys
 * (section 3 "Spacetime Sparse Attention").  Strides are in elements for the
 * batch, head and token dimensions; the head_dim stride is 1.
 *
 * Blocks.  Query block i holds tokens [i*b, min((i+1)*b, L_q)); key block j
 * holds [j*b, min((j+1)*b, L_k)); n_q = ceil(L_q/b), n_k = ceil(L_k/b).
 * Blocks are not aligned to the text/reference/current boundaries (section 5
 * "Original-order block partition").
 *
 * Memory and streams.  Every pointer passed to a device call is a device
 * pointer owned by the caller.  The library never allocates or frees device
 * memory, never synchronises, and keeps no pointer after a call returns.  Each
 * device call validates all of its arguments on the host first; a non-OK
 * status means nothing was enqueued.  After validation, work is enqueued on
 * `stream` (a hipStream_t; NULL is the default stream) and the call returns
 * without waiting.  A fault inside a kernel surfaces at the caller's next
 * synchronisation.  Outputs must not alias inputs.  Calls are reentrant; the
 * last-error text is per thread.
 */
#ifndef SPARSTAR_H
#define SPARSTAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSTAR_OK = 0,
  SPARSTAR_ERR_NULL = 1,        /* a required pointer is NULL                              */
  SPARSTAR_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree                */
  SPARSTAR_ERR_UNSUPPORTED = 3, /* valid but not built: head_dim, block, dtype, device     */
  SPARSTAR_ERR_LAYOUT = 4,      /* stride or pointer alignment not supported               */
  SPARSTAR_ERR_DENSITY = 5,     /* density not in (0, 1]                                  */
  SPARSTAR_ERR_CAPACITY = 6,    /* an output buffer is smaller than the result             */
  SPARSTAR_ERR_HIP = 7          /* the HIP runtime reported an error                       */
} sparstar_status;

typedef enum { SPARSTAR_BF16 = 0, SPARSTAR_F32 = 1 } sparstar_dtype;

/* Which key blocks stay dense and which are ranked (section 5 "Clip-Dependent
 * Retained and Selectable Blocks"; appendix A.7 "Later-clip schedule").
 * LATER_CLIP (clip c >= 2): the blocks touching the text stay; reference and
 *   current blocks are ranked jointly under one budget.
 * FIRST_CLIP (clip 1): the blocks touching the text or the reference (for clip
 *   1 the final image-pyramid scale) stay; only the rest are ranked.
 * In both the retained set is the prefix of key blocks [0, r) and the ranked
 * candidates are [r, n_k). */
typedef enum { SPARSTAR_POLICY_LATER_CLIP = 0, SPARSTAR_POLICY_FIRST_CLIP = 1 } sparstar_policy;

typedef struct {
  int32_t batch;          /* B >= 0                                                     */
  int32_t heads;          /* H >= 0                                                     */
  int32_t head_dim;       /* D: 64 or 128                                               */
  int32_t block;          /* b: 64, 128 or 256, the same for query and key blocks
                             (128 deployed; 64 and 256 from appendix D.2)                */
  int64_t len_q;          /* L_q >= 0: current-scale tokens (queries, last keys)        */
  int64_t len_text;       /* L_text >= 0                                                */
  int64_t len_ref;        /* L_ref >= 0: the preceding clip's final scale               */
  int32_t dtype;          /* sparstar_dtype of Q, K, V                                  */
  int32_t out_dtype;      /* sparstar_dtype of the attention output                     */
  float softmax_scale;    /* sigma > 0, finite (1/sqrt(D) in the workloads)            */
  int32_t reserved;       /* must be 0                                                  */
  int64_t q_stride[3];    /* element strides of Q over (batch, head, token)            */
  int64_t k_stride[3];    /* ... of K                                                   */
  int64_t v_stride[3];    /* ... of V                                                   */
  int64_t o_stride[3];    /* ... of the output                                          */
} sparstar_problem;

/* ---------------- host-only helpers: no HIP call, usable without a GPU ---------------- */

/* Validates the problem description alone (sizes, dtypes, strides, scale). */
sparstar_status sparstar_check_problem(const sparstar_problem* p);

/* n_q = ceil(L_q/b) and n_k = ceil(L_k/b); -1 if the problem is invalid. */
int64_t sparstar_num_q_blocks(const sparstar_problem* p);
int64_t sparstar_num_k_blocks(const sparstar_problem* p);

/* Number r of retained key blocks under `policy` (the prefix [0, r)); -1 if invalid. */
int64_t sparstar_num_retained(const sparstar_problem* p, int32_t policy);

/* Budget k for n_candidates ranked blocks at `density` (section 5 "Clip-Dependent
 * Retained and Selectable Blocks"): k = ceil(density*n - 1e-6) clamped to [1, n],
 * and 0 if n == 0; -1 if density is not in (0, 1] or n < 0. */
int64_t sparstar_budget(int64_t n_candidates, double density);

/* Key blocks listed per query block: r + k; -1 if invalid. */
int64_t sparstar_blocks_per_row(const sparstar_problem* p, double density, int32_t policy);

/* Entries of col_idx written by sparstar_select_blocks: B*H*n_q*(r + k); -1 if invalid. */
int64_t sparstar_select_nnz(const sparstar_problem* p, double density, int32_t policy);

const char* sparstar_status_string(sparstar_status s);

/* Detail text of the last non-OK status returned on this thread ("" if none). */
const char* sparstar_last_error(void);

/* ---------------- device calls: pointers are device pointers; async on `stream` ------- */

/* Steps 1-2 (section 5 "Original-order block partition", "Per-head aggregated
 * query-key score").
 *   q, k     : inputs in p->dtype with p's strides.
 *   q_pool   : out, float32 [B, H, n_q, D] contiguous: q_pool[i] = (1/b) * sum of the
 *              real tokens of query block i (a partial last block is zero-padded
 *              and still divided by b).
 *   k_pool   : out, float32 [B, H, n_k, D] contiguous, likewise for key blocks.
 *   scores   : out, float32 [B, H, n_q, n_k] contiguous: sigma * <q_pool_i, k_pool_j>.
 * Sums and products are float32. */
sparstar_status sparstar_pool_score(const sparstar_problem* p, const void* q, const void* k,
                                    float* q_pool, float* k_pool, float* scores, void* stream);

/* Step 2 without the scores: the block means of sparstar_pool_score only (same
 * arguments and results for q_pool and k_pool, bit for bit), for
 * sparstar_score_select. */
sparstar_status sparstar_pool_blocks(const sparstar_problem* p, const void* q, const void* k,
                                     float* q_pool, float* k_pool, void* stream);

/* Steps 2b and 3 fused (section 5 "Per-head aggregated query-key score" and
 * "Clip-Dependent Retained and Selectable Blocks"; the scope's "score-then-select
 * that never materialises S"): the block lists of sparstar_select_blocks computed
 * from the block means, with no score matrix in memory.  For each head and strip
 * of 32 query blocks the scores are formed in LDS, in the same float32 operations
 * as sparstar_pool_score, so row_ptr and col_idx are the same, bit for bit, as
 * sparstar_pool_score followed by sparstar_select_blocks.
 *   q_pool, k_pool : in, float32 [B, H, n_q, D] / [B, H, n_k, D] contiguous
 *                    (sparstar_pool_blocks or sparstar_pool_score).
 *   density, policy, row_ptr, col_idx, col_idx_capacity : as sparstar_select_blocks.
 * A strip's scores must fit LDS: n_k at most 1,152 (SPARSTAR_ERR_UNSUPPORTED beyond). */
sparstar_status sparstar_score_select(const sparstar_problem* p, const float* q_pool, const float* k_pool,
                                      double density, int32_t policy, int32_t* row_ptr, int32_t* col_idx,
                                      int64_t col_idx_capacity, void* stream);

/* Step 3 (section 5 "Clip-Dependent Retained and Selectable Blocks" and
 * "Forward-Only Sparse Execution"; appendix A.7).  For every row
 * r = (b*H + h)*n_q + i the listed blocks are the retained prefix [0, r_keep)
 * followed by the k best candidates of scores[b, h, i, r_keep:n_k], best meaning
 * the larger score, exactly equal scores going to the lower block index; the
 * list is ascending.  This is the forward-only BlockMask (kv_num_blocks,
 * kv_indices) in CSR form.
 *   scores   : in, float32 [B, H, n_q, n_k] contiguous (as written by pool_score).
 *   row_ptr  : out, int32 [B*H*n_q + 1]; row_ptr[r] = r * (r_keep + k).
 *   col_idx  : out, int32 [col_idx_capacity]; the first sparstar_select_nnz entries
 *              are written.  SPARSTAR_ERR_CAPACITY if the capacity is smaller.
 * One wavefront ranks a row with its candidates held in registers: at most 4,096
 * candidate blocks per row (n_k - r_keep), SPARSTAR_ERR_UNSUPPORTED beyond.  The
 * total nnz must fit int32 (SPARSTAR_ERR_SHAPE otherwise).
 * NaN scores are not supported (their rank is unspecified). */
sparstar_status sparstar_select_blocks(const sparstar_problem* p, const float* scores,
                                       double density, int32_t policy, int32_t* row_ptr,
                                       int32_t* col_idx, int64_t col_idx_capacity, void* stream);

/* Bytes of device workspace sparstar_bsa_fwd and dense_attn_fwd take for their row
 * queues (256: the counters of the per-XCD queues); -1 if the problem is invalid. */
int64_t sparstar_bsa_workspace_bytes(const sparstar_problem* p);

/* Step 4 (section 5 "Forward-Only Sparse Execution", "Complexity and Scope").
 * Each query t of block i gets o_t = sum_s softmax_s(sigma * q_t.k_s) v_s over the
 * real key tokens s (< L_k) of the blocks col_idx[row_ptr[r] .. row_ptr[r+1]),
 * r = (b*H + h)*n_q + i.  Entries outside [0, n_k) and positions outside
 * [0, col_idx_len) are skipped; a row with no valid block gets o = 0 and
 * lse = -inf.  A block listed twice counts twice.
 *   q, k, v  : inputs in p->dtype.
 *   row_ptr  : in, int32 [B*H*n_q + 1];  col_idx: in, int32 [col_idx_len].
 *   out      : out, p->out_dtype with p->o_stride; rows >= L_q are not written.
 *   lse      : out, nullable, float32 [B, H, L_q] contiguous: sigma*max + log(sum exp).
 *   workspace: nullable device buffer of at least sparstar_bsa_workspace_bytes bytes,
 *              owned by the caller (SPARSTAR_ERR_CAPACITY if smaller).  With it, a
 *              persistent grid of as many workgroups as fit on the GPU at once takes
 *              the rows from per-XCD queues with atomic counters, which the call
 *              sets itself (a kernel, no memset), and a workgroup whose XCD has no
 *              rows left takes rows from the other XCDs' queues; two calls must not
 *              share a workspace while either runs.  With NULL (and any
 *              workspace_bytes), or when the problem has fewer rows than two
 *              rounds of the persistent grid per XCD, one workgroup per row, handed
 *              to the XCDs by the hardware dispatcher (the workspace is then not
 *              touched).  The outputs are the same, bit for bit, either way.
 * bf16 inputs with D = 128 run on bf16 MFMA with float32 softmax and accumulation
 * for every block size (64, 128, 256: the block sizes of appendix D.2 "Block-Size
 * Ablation").
 * D = 64 and float32 inputs run a float32 kernel (sparstar_attention_kernel tells
 * which), which ignores the workspace. */
sparstar_status sparstar_bsa_fwd(const sparstar_problem* p, const void* q, const void* k,
                                 const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                                 int64_t col_idx_len, void* out, float* lse, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Which kernel sparstar_bsa_fwd, sparstar_bsa_fwd_balanced and dense_attn_fwd run for a
 * problem: SPARSTAR_KERNEL_MFMA_BF16 for bf16 inputs with head_dim 128 whose in-head
 * byte offsets (L + 256 tokens at the largest token stride) stay below 2^31;
 * SPARSTAR_KERNEL_F32 (a float32 kernel, one thread per query: correct, not tuned)
 * for every other valid problem, bf16 inputs with head_dim 64 included; -1 if the
 * problem is invalid.  Host only. */
typedef enum { SPARSTAR_KERNEL_MFMA_BF16 = 0, SPARSTAR_KERNEL_F32 = 1 } sparstar_kernel;
int32_t sparstar_attention_kernel(const sparstar_problem* p);

/* Dense attention forward (every key block of every row): the density-1 baseline
 * that the sparse operator is compared with (section 6 "End-to-end efficiency").
 * Arguments, workspace included, as for sparstar_bsa_fwd without the block lists. */
sparstar_status dense_attn_fwd(const sparstar_problem* p, const void* q, const void* k,
                               const void* v, void* out, float* lse, void* workspace,
                               int64_t workspace_bytes, void* stream);

/* Bytes of device workspace sparstar_bsa_fwd_balanced needs: 256 bytes of row-queue
 * counters followed by the row order, 4 * B*H*S*ceil(n_q/S) bytes, with S = 4 segments
 * per head at blocks 128 and 256 when B*H is even, and S = 8 otherwise; -1 if the
 * problem is invalid. */
int64_t sparstar_balance_workspace_bytes(const sparstar_problem* p);

/* sparstar_bsa_fwd for block lists of uneven length (section 5 "Forward-Only Sparse
 * Execution": the lists are per query block and their lengths are the caller's).
 * The attention runs the query blocks of a head in S contiguous segments of
 * ceil(n_q/S) blocks, one per XCD (S = 4 at blocks 128 and 256 with an even B*H: two
 * heads at a time; S = 8 otherwise: one head at a time), heads in order.  Here the rows of
 * each segment are first ordered by list length, longest first and stably (equal lengths
 * keep their order), and the persistent workgroups take rows from per-XCD queues with
 * atomic counters: a workgroup whose XCD's queue is empty takes rows from the other
 * XCDs' queues, so no XCD idles while another still has rows.  `workspace` is a device
 * buffer of at least sparstar_balance_workspace_bytes, owned by the caller; the call
 * sets the counters itself (a kernel, no memset).  On return bytes [0, 256) hold the
 * counters and from byte 256 on the order: entry (b*H + h)*S*ceil(n_q/S) + x*ceil(n_q/S) + m
 * is the query block of the m-th row of segment x, -1 past the segment's end.  Every row
 * is computed exactly as by sparstar_bsa_fwd: the outputs are the same, bit for bit.  The
 * queues and the order are used by the bf16 MFMA kernel; the float32 kernel (see
 * sparstar_attention_kernel) runs the rows in their natural order, and the workspace is
 * still written.  SPARSTAR_ERR_CAPACITY if the workspace is too small.
 * Two calls must not share a workspace while either runs. */
sparstar_status sparstar_bsa_fwd_balanced(const sparstar_problem* p, const void* q, const void* k,
                                          const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                                          int64_t col_idx_len, void* out, float* lse, void* workspace,
                                          int64_t workspace_bytes, void* stream);

/* sparstar_bsa_fwd_balanced without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The row queues' counters and the row order
 * live in a scratch array the library holds on each device (1 MiB, kept until the
 * process ends; its address is looked up once per device, on the first call there);
 * the call allocates nothing.  Problems whose queues and order need more than that
 * (sparstar_balance_workspace_bytes > 1,048,576, i.e. B*H*S*ceil(n_q/S) above 262,080
 * rows) are refused with SPARSTAR_ERR_CAPACITY before anything is enqueued.  Every
 * call on one device shares that device's scratch, which keeps the last call's
 * contents (the call sets the counters itself): calls that overlap on one device,
 * on different streams or from different threads, race and must not be made.
 * Arguments, results and errors otherwise as sparstar_bsa_fwd_balanced; the outputs
 * are the same, bit for bit. */
sparstar_status sparstar_bsa_fwd_balanced_noalloc(const sparstar_problem* p, const void* q, const void* k,
                                                  const void* v, const int32_t* row_ptr,
                                                  const int32_t* col_idx, int64_t col_idx_len, void* out,
                                                  float* lse, void* stream);

/* ---------------- retained attention mass (the pages' quality measure of a selection) ---
 * Section 4 "Analysis" (Figure 3; "Pattern Persistence across Clip Boundaries")
 * and section 1 measure a selection by the share of each query's dense softmax
 * mass it keeps, against the token-wise Top-K bound, the exact block oracle, a
 * sliding window and random blocks.  With w_ts = exp(sigma*q_t.k_s - lse_t) the
 * dense attention weight of query t on real key s (lse from dense_attn_fwd):
 *   - the exact block oracle is sparstar_select_blocks fed the block mass below;
 *   - a sliding window is sparstar_select_blocks fed sparstar_window_scores;
 *   - random blocks are sparstar_select_blocks fed caller-drawn uniform numbers. */

/* M[b, h, i, j] = sum over the real queries t of query block i and the real keys s of
 * key block j of w_ts.  Row i sums to the number of real queries of block i.
 *   q, k : inputs in p->dtype with p's strides (v and out strides are not used).
 *   lse  : in, float32 [B, H, L_q] contiguous (dense_attn_fwd's lse output).
 *   mass : out, float32 [B, H, n_q, n_k] contiguous.
 * bf16 with D = 128 and b = 128 runs on bf16 MFMA (float32 exp2 and sums); other
 * shapes on a float32 kernel.  Deterministic (fixed summation order). */
sparstar_status sparstar_block_mass(const sparstar_problem* p, const void* q, const void* k,
                                    const float* lse, float* mass, void* stream);

/* Mean retained mass per query block of a block selection:
 * row_mass[r] = sum over the entries j of row r (r = (b*H + h)*n_q + i) of mass[r, j],
 * divided by the real queries of block i.  Entries outside [0, n_k) and positions
 * outside [0, col_idx_len) are skipped; a block listed twice counts twice.
 *   mass     : in, float32 [B, H, n_q, n_k] (sparstar_block_mass).
 *   row_ptr  : in, int32 [B*H*n_q + 1];  col_idx: in, int32 [col_idx_len].
 *   row_mass : out, float32 [B*H*n_q]. */
sparstar_status sparstar_selection_mass(const sparstar_problem* p, const float* mass,
                                        const int32_t* row_ptr, const int32_t* col_idx,
                                        int64_t col_idx_len, float* row_mass, void* stream);

/* Sliding-window scores: scores[b, h, i, j] = -|(j*b + b/2) - (L_text + L_ref + i*b + b/2)|,
 * minus the distance in key-sequence position between the centres of key block j and
 * query block i (query t is key L_text + L_ref + t).  Through sparstar_select_blocks
 * every query block gets the k candidate blocks nearest to it, equal distances to the
 * lower index.   scores: out, float32 [B, H, n_q, n_k] contiguous. */
sparstar_status sparstar_window_scores(const sparstar_problem* p, float* scores, void* stream);

/* Token-wise Top-K bound for listed queries: out[n] = sum of w_ts over the key tokens
 * s < keep_tokens plus the k_tokens largest w_ts over the key tokens s >= keep_tokens
 * (all of them if fewer), for query index rows[n] = (b*H + h)*L_q + t.  With
 * keep_tokens = (retained blocks)*b and k_tokens = k*b this bounds the mass any
 * selection of k candidate blocks keeps for that query.
 *   q, k : inputs;  lse: in, float32 [B, H, L_q] (dense_attn_fwd).
 *   rows : in, int64 [n_rows], 8-byte aligned; an index outside [0, B*H*L_q) gives NaN.
 *   out  : out, float32 [n_rows].
 * Weights in float32; the k-th largest is found exactly on their float32 values. */
sparstar_status sparstar_token_topk_mass(const sparstar_problem* p, const void* q, const void* k,
                                         const float* lse, const int64_t* rows, int64_t n_rows,
                                         int64_t keep_tokens, int64_t k_tokens, float* out,
                                         void* stream);

/* ---------------- measurement helper (not a step of the method) --------------------------
 * The bf16 matrix-core rate the GPU sustains on operands like the attention's, against
 * which the attention's own rate can be read (its published peak assumes a clock the
 * part does not hold under this load).  Each lane of two 4-wavefront workgroups per CU
 * runs eight independent chains of v_mfma_f32_32x32x16_bf16 (the attention's
 * instruction) on operands drawn from a counter hash, uniform in [-2, 2), a new operand
 * pair for every instruction; fixed operands would draw less power and overstate it. */

/* Floats the sink of sparstar_mfma_probe must hold on the current device (256 per
 * workgroup, two workgroups per CU); -1 if the device cannot be queried. */
int64_t sparstar_mfma_probe_sink_len(void);

/* One launch of `rounds` rounds (64 instructions per wavefront each) on `stream`.
 *   sink : out, device float32 [sink_len], one value per lane (keeps the chains live).
 *   flops: out, host, nullable: the multiply-add flops of the launch (2*32*32*16 per
 *          instruction); divide by the launch time for the rate.
 * SPARSTAR_ERR_SHAPE if rounds < 1, SPARSTAR_ERR_NULL for a NULL sink,
 * SPARSTAR_ERR_LAYOUT if it is not 4-byte aligned, SPARSTAR_ERR_CAPACITY if sink_len
 * is below sparstar_mfma_probe_sink_len(). */
sparstar_status sparstar_mfma_probe(int32_t rounds, float* sink, int64_t sink_len, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSTAR_H */
