/*
 * nsa.h -- C ABI of the MI355X (gfx950) native-sparse-attention hot path.
 *
 * The path, as the source pages describe it:
 *   1. mean-pool keys into overlapping windows (32 tokens, stride 16)
 *      [NOSA-1B core components, component 1 "Key compressor"];
 *   2. score each query against the compressed keys and sum the softmax
 *      probabilities over the query heads of a GQA group, then max-pool the
 *      window scores onto 64-token blocks
 *      [NOSA-1B core components, component 3; NOSA-1B source analysis part 3,
 *      "beyond the kernel"];
 *   3. mean-pool the per-token CIS importance scores over the same windows,
 *      varlen by cu_seqlens, dividing by the count of valid tokens
 *      [NOSA-1B source analysis part 3, grid / block-load / varlen-mask
 *      sections; NOSA-1B core components, component 2];
 *   4. keep the init and local blocks and the top-k of the rest, indices sorted
 *      [NOSA-1B source analysis part 3, "beyond the kernel"; component 3];
 *   5. GQA-grouped attention over only the selected blocks, optionally with CIS-
 *      scaled values and the ones-value normaliser
 *      [NOSA-1B core components, decode-stage section; TileLang NSA, section 2].
 *   The three-branch NSA prefill (compressed, selected and sliding-window
 *   branches summed with gates) follows DeepSeek NSA with Triton, section 1.1.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL is the default stream) and the call returns at once.
 *   - Packed variable-length batches: sequence b occupies rows
 *     cu_seqlens[b] .. cu_seqlens[b+1]-1 of a packed tensor.  cu_seqlens arrays
 *     are device int32 [batch+1], non-decreasing, starting at 0.  The max_*
 *     sizes passed by value are host-side upper bounds used to size the grid;
 *     a smaller real size is fine, a larger one is undefined behaviour.
 *   - Layouts (row-major, innermost last):
 *       Q          [rows, heads, head_dim]       (decode: rows = batch)
 *       K, V       [N_k, kv_heads, head_dim]
 *       K_c        [N_c, kv_heads, head_dim]     window c of sequence b at row
 *                                                cu_seqlens_c[b] + c
 *       cis        [N_k, kv_heads] float32;  cis_pooled [N_c, kv_heads] float32
 *       block_scores [rows, kv_heads, n_blocks_max] float32
 *       indices    [rows, kv_heads, k] int32, block ids local to the sequence,
 *                  ascending, -1 padded
 *   - Window c of a sequence of length L covers its tokens
 *     stride*c .. stride*c+kernel-1 that exist (< L).  The number of windows of
 *     sequence b is cu_seqlens_c[b+1]-cu_seqlens_c[b]; the usual choice is the
 *     full-window count floor((L-kernel)/stride)+1 (0 when L < kernel).
 *   - A query at position t (0-based, within its sequence) sees window c when
 *     stride*c+kernel-1 <= t, and block i when 0 <= block_size*i <= t; inside a
 *     selected block only tokens j <= t are attended.  Decode queries sit at
 *     t = L-1.  Prefill rows (cu_seqlens_q given) of sequence b sit at
 *     t = (row - cu_seqlens_q[b]) + (L_k - L_q).
 *   - softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   - Supported: head_dim 128; heads/kv_heads in {1, 2, 4, 8, 16}; kernel 32,
 *     stride 16 for the scoring paths (pooling accepts any kernel >= stride >= 1);
 *     block_size 64.  Others return NSA_ERR_UNSUPPORTED without launching.
 *   - Workspaces are caller-allocated device memory of at least the size the
 *     matching *_workspace_size query returns.  They need no initialisation:
 *     every call writes each workspace byte it later reads.  A workspace can be
 *     reused by later calls on the same stream; calls that share one workspace
 *     must not run concurrently.
 *   - Errors: every entry point validates its arguments on the host before
 *     launching and returns a non-zero nsa_status on failure; nsa_last_error()
 *     then describes it (thread-local string, valid until the next call on
 *     that thread).  NSA_ERR_HIP reports a launch error from hipGetLastError.
 *     Preconditions NOT checked on the release path (undefined behaviour if
 *     broken): cu_seqlens contents, unique block ids within one index row,
 *     finite inputs; nsa_set_debug_checks(1) checks the first two (and NaN-free
 *     block scores) on the device.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nsa_status {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARG = 1,
  NSA_ERR_UNSUPPORTED = 2,
  NSA_ERR_WORKSPACE = 3,
  NSA_ERR_HIP = 4
} nsa_status;

typedef enum nsa_dtype {
  NSA_F32 = 0,  /* IEEE float32 */
  NSA_BF16 = 1  /* bfloat16 */
} nsa_dtype;

/* Thread-local text of the last error (empty string after a successful call). */
const char* nsa_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t nsa_version(void);

/*
 * nsa_set_debug_checks -- debug mode for the whole process (off by default);
 * returns the previous setting.  While on, every entry point that takes
 * sequence offsets or block lists first checks on the device the preconditions
 * the release path takes on trust: each cu_seqlens array starts at 0 and never
 * decreases, no sequence is longer than max_seqlen_k, no sequence has more query
 * rows than keys or more windows than cover its tokens, the ids of one index row
 * are distinct, block scores given to nsa_select_topk hold no NaN.  The call
 * then waits for those checks (the only synchronisation in the library) and
 * returns NSA_ERR_INVALID_ARG, naming the broken precondition, without
 * launching its work.  [The varlen layout is the one NOSA-1B source analysis
 * part 3 masks by (sequence b spans rows cu[b] .. cu[b+1]-1); distinct ids
 * follow the block lists of TileLang NSA, section 2.]  Not for graph capture.
 */
int32_t nsa_set_debug_checks(int32_t on);

/*
 * nsa_profile_next_launch -- measurement hook (not part of the method).  Arms
 * the next launch, on the calling host thread, of one kernel kind so that it
 * records `start` and `stop` at the kernel's own begin and end
 * (hipExtLaunchKernelGGL); the request is consumed by that launch.  Kinds:
 * 0 pooling (nsa_compress_k, nsa_cis_mean_pool_varlen), 1 compressed-key
 * logits (with the decode window refresh), 2 block scores and top-k
 * selection, 3 selected attention, 4 merge of split partial states (decode),
 * 5 compressed-attention normaliser pass (prefill), 6 compressed-attention
 * output and block-score pass (prefill), 7 sliding-window attention (prefill,
 * with the gated sum in nsa_prefill_step), 8 block copies from host memory
 * (nsa_decode_step_offload), 9 block-mask attention, 10 selected-attention
 * backward dq, 11 its dk and dv, 12 its delta and per-block row lists (the
 * first of those four launches), 13 the sum of its key-block dq partial states.  The events are owned by the caller
 * and must have timing enabled; a launch made during stream capture must not
 * be armed.
 */
typedef enum nsa_kernel_kind {
  NSA_KERNEL_POOL = 0,
  NSA_KERNEL_LOGITS = 1,
  NSA_KERNEL_BLOCK_SCORES = 2,
  NSA_KERNEL_SELECTED_ATTN = 3,
  NSA_KERNEL_COMBINE = 4,
  NSA_KERNEL_COMPRESSED_LSE = 5,
  NSA_KERNEL_COMPRESSED_ATTN = 6,
  NSA_KERNEL_WINDOW_ATTN = 7,
  NSA_KERNEL_FETCH = 8,
  NSA_KERNEL_BLOCKMASK_ATTN = 9,
  NSA_KERNEL_SELECTED_BWD_DQ = 10,
  NSA_KERNEL_SELECTED_BWD_DKDV = 11,
  NSA_KERNEL_SELECTED_BWD_LISTS = 12,
  NSA_KERNEL_SELECTED_BWD_DQ_SUM = 13,
  NSA_KERNEL_BLOCK_LISTS = 14
} nsa_kernel_kind;
nsa_status nsa_profile_next_launch(int32_t kernel_kind, hipEvent_t start, hipEvent_t stop);

/*
 * nsa_window_count -- number of compressed windows of one sequence, the count a
 * caller puts into cu_seqlens_c.
 * [NOSA-1B source analysis part 3: the avg_pool1d consistency check (windows
 *  that lie wholly inside the sequence) and the masked block load (a window
 *  reaching past the end keeps only its valid tokens, divided by their count).]
 *   tail_mode 0: full windows only, floor((length - kernel) / stride) + 1, and 0
 *                when length < kernel (the default of every scoring path);
 *   tail_mode 1: windows until every token is covered, the smallest n with
 *                stride * (n - 1) + kernel >= length (1 when 0 < length <=
 *                kernel, 0 when length == 0); the last ones are partial.
 * The pooling entry points take the window count of each sequence from
 * cu_seqlens_c, so the tail mode is chosen by building cu_seqlens_c from this
 * function.  Returns -1 when length < 0, kernel < 1, stride < 1 or tail_mode is
 * neither 0 nor 1.  Host function; touches no device state.
 */
int32_t nsa_window_count(int32_t length, int32_t kernel, int32_t stride, int32_t tail_mode);

/*
 * nsa_compress_k -- mean-pool keys (or values) into compressed windows.
 * [NOSA-1B core components, component 1: CompressK, 32-token windows, stride 16,
 *  one mean per window.]
 *   x      [N, heads, head_dim] of dtype x_dtype
 *   x_c    [N_c, heads, head_dim] of dtype xc_dtype (written); float32 keeps the
 *          full-precision mean, bfloat16 rounds it to nearest even.
 *   max_windows  >= every sequence's window count.
 * Each window is the sum of its valid tokens divided by their number, 0 if none.
 */
nsa_status nsa_compress_k(const void* x, nsa_dtype x_dtype, void* x_c, nsa_dtype xc_dtype,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_c,
                          int32_t batch, int32_t max_windows, int32_t heads,
                          int32_t head_dim, int32_t kernel, int32_t stride,
                          hipStream_t stream);

/*
 * nsa_cis_mean_pool_varlen -- sliding-window mean of per-token importance scores.
 * [NOSA-1B source analysis part 3: grid (head, batch, window), masked load of the
 *  window, sum divided by the valid count; NOSA-1B core components, component 2:
 *  kernel 32 / stride 16, aligned with the key compressor.]
 *   cis        [N, heads] float32
 *   cis_pooled [N_c, heads] float32 (written)
 */
nsa_status nsa_cis_mean_pool_varlen(const float* cis, float* cis_pooled,
                                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_c,
                                    int32_t batch, int32_t max_windows, int32_t heads,
                                    int32_t kernel, int32_t stride, hipStream_t stream);

/*
 * nsa_compressed_scores -- block scores of decode queries (one query per
 * sequence, at t = L-1).
 * [NOSA-1B core components, component 3, stage 1: attention of the query against
 *  the compressed keys gives block scores; NOSA-1B source analysis part 3, "beyond
 *  the kernel": window scores max-pooled to blocks and fused with the pooled CIS.]
 *   q            [batch, heads, head_dim], dtype q_dtype
 *   k_c          [N_c, kv_heads, head_dim], dtype kc_dtype
 *   cis_pooled   nullable [N_c, kv_heads] float32; with it the block score gains
 *                cis_weight * (max of cis_pooled over the block's windows)
 *   block_scores [batch, kv_heads, n_blocks_max] float32 (written), with
 *                n_blocks_max = ceil(max_seqlen_k / block_size); entries past a
 *                sequence's own block count are written as 0
 *   window_probs nullable [batch, kv_heads, max_windows] float32 (written): the
 *                group-summed probabilities, 0 past a sequence's window count
 *   For query head h (group g = h / (heads/kv_heads)): P_h = softmax over visible
 *   windows of scale * q_h . K_c[c]; P_g = sum of P_h over the group; block score
 *   = max of P_g over windows overlapping the block (0 if none).
 *   workspace: nsa_compressed_scores_workspace_size(...) bytes.
 */
size_t nsa_compressed_scores_workspace_size(int32_t batch, int32_t max_seqlen_k, int32_t heads,
                                            int32_t kv_heads, int32_t kernel, int32_t stride);
nsa_status nsa_compressed_scores(const void* q, nsa_dtype q_dtype, const void* k_c,
                                 nsa_dtype kc_dtype, const float* cis_pooled, float cis_weight,
                                 float* block_scores, float* window_probs,
                                 const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_c,
                                 int32_t batch, int32_t max_seqlen_k, int32_t heads,
                                 int32_t kv_heads, int32_t head_dim, int32_t kernel,
                                 int32_t stride, int32_t block_size, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nsa_select_topk -- top-k block selection with forced init and local blocks.
 * [NOSA-1B source analysis part 3, "beyond the kernel": init and local blocks are
 *  kept, other positions compete by score, top-k picks the ids, ids are sorted;
 *  NOSA-1B core components, component 3: k = 64.]
 *   block_scores [rows, kv_heads, n_blocks_max] float32, NaN-free
 *   indices      [rows, kv_heads, k] int32 (written)
 *   cu_seqlens_q NULL: decode, rows = batch, t = L_b - 1.  Otherwise prefill rows.
 *   Eligible blocks: block_size*i <= t.  Forced: the first n_init and the last
 *   n_local eligible blocks (n_init + n_local <= k).  The other k - |forced|
 *   places go to the best-scoring eligible blocks, ties to the lower id.  Output
 *   ascending, padded with -1 when fewer than k blocks are eligible.
 *   rows_total: number of rows (batch for decode; cu_seqlens_q[batch] otherwise).
 */
nsa_status nsa_select_topk(const float* block_scores, int32_t* indices,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                           int32_t kv_heads, int32_t n_blocks_max, int32_t k, int32_t n_init,
                           int32_t n_local, int32_t block_size, hipStream_t stream);

/*
 * nsa_selected_attn_fwd -- attention of each query row over its selected blocks.
 * [NOSA-1B core components, decode stage: sparse FlashAttention over the topk_idx
 *  blocks, values scaled by CIS and a ones-value normaliser; TileLang NSA,
 *  section 2: BlockIndices[b, t, h_kv, :], block start id*64 used when
 *  0 <= start <= t, query heads of one KV group share the KV blocks.]
 *   q, out   [rows, heads, head_dim] of `dtype` (out written)
 *   k, v     [N_k, kv_heads, head_dim] of `dtype`
 *   indices  [rows, kv_heads, k_sel] int32
 *   cis      nullable [N_k, kv_heads] float32.  NULL: out = softmax(s) . V.
 *            Given: out = sum_j p_j cis_j v_j / sum_j p_j cis_j (the CIS-scaled
 *            values divided by the same attention over all-ones values).
 *   lse      nullable [rows, heads] float32 (written): natural log of the
 *            normaliser sum_j exp(s_j) (times cis_j in CIS mode); -inf when the
 *            row sees no key (its output row is then 0).
 *   cu_seqlens_q NULL: decode (rows = batch, t = L_b - 1); else prefill rows.
 *   workspace: decode rows: nsa_selected_attn_workspace_size(..., decode=1)
 *            bytes, required.  Prefill rows: optional.  NULL or 0 bytes (or
 *            float32 inputs): one workgroup per (row, KV head) gathers the
 *            row's blocks.  Given with at least
 *            nsa_selected_attn_workspace_size(..., decode=0) bytes
 *            (rows * heads * k_sel * 264 + rows * kv_heads * k_sel * 10
 *            bytes, 16-byte aligned) and bf16 inputs: key-block stationary --
 *            the valid places of every (sequence, KV head, 1024 query rows)
 *            are listed by block, then one workgroup per (sequence, KV head,
 *            1024 query rows, listed 64-key block) attends the rows listing
 *            the block and writes their partial state (bf16 output, fp32 max
 *            and sum) at the row's place; a merge kernel combines each row's
 *            places.  This path also needs every L_b <= max_seqlen_k and at
 *            most 8192 blocks per sequence (else NSA_ERR_UNSUPPORTED).  Between
 *            0 and the queried size: NSA_ERR_WORKSPACE.  An id listed twice
 *            in one row counts once on this path and twice on the other (ids
 *            of a row must be unique either way).
 */
size_t nsa_selected_attn_workspace_size(int32_t rows_total, int32_t heads, int32_t kv_heads,
                                        int32_t head_dim, int32_t k_sel, int32_t decode);
nsa_status nsa_selected_attn_fwd(const void* q, const void* k, const void* v, nsa_dtype dtype,
                                 const int32_t* indices, int32_t k_sel, const float* cis,
                                 void* out, float* lse, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t batch, int32_t rows_total,
                                 int32_t max_seqlen_k, int32_t heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t block_size, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nsa_selected_attn_bwd -- gradient of nsa_selected_attn_fwd (plain softmax,
 * no CIS) over prefill rows.
 * [DeepSeek NSA with Triton, introduction and section 2.3: the method is
 *  trained end to end, its kernels wrapped as a trainable module; the pages
 *  print no backward, so this is the exact gradient of the forward above.]
 *   q, out, d_out [rows, heads, 128] bf16: the forward's queries, its output
 *                 and the upstream gradient of that output
 *   k, v          [N_k, kv_heads, 128] bf16
 *   lse           [rows, heads] float32: the forward's natural-log normaliser
 *   indices       [rows, kv_heads, k_sel] int32, the forward's (ids of one row
 *                 unique; -1 and ids with 64*id > t are skipped)
 *   cu_seqlens_q, cu_seqlens_k (required): row r of sequence b sits at
 *                 t = (r - cu_q[b]) + (L_b - Lq_b); every L_b <= max_seqlen_k.
 *   dq            [rows, heads, 128] float32, written
 *   dk, dv        [N_k, kv_heads, 128] float32, written in full (0 for keys no
 *                 row attends to)
 *   Per head over the row's keys J: dV_J += p dO^T; ds = p*(V_J dO - dO.O);
 *   dq = scale ds K_J; dK_J += scale ds q^T.  dk and dv are gathered per
 *   (sequence, KV head, block) over the rows that list the block, up to 512
 *   rows per workgroup; a block listed by more rows has its chunk sums added
 *   with fp32 atomics.  The row lists are built with atomics too, so the
 *   summation order of dk and dv may change between calls (fp32 rounding only).
 *   workspace: device memory, 16-byte aligned.  With
 *   nsa_selected_attn_bwd_workspace_size(...) bytes dq is computed key-block
 *   stationary, as the forward given a workspace: per (sequence, KV head,
 *   listed 64-key block, 1024 rows) the block's share of dq of every listing
 *   row is written as bf16 at (row, place, head) (rows * heads * k_sel * 256
 *   bytes of the workspace, and rows * kv_heads * k_sel * 10 bytes for the
 *   block lists; at most 8192 blocks per sequence, else dq runs row by row),
 *   then the valid places of each (row, head) are summed in
 *   fp32.  Any size from nsa_selected_attn_bwd_workspace_size_min(...) up to
 *   that computes dq with one workgroup per (row, KV head).  Less:
 *   NSA_ERR_WORKSPACE.
 *   Returns NSA_ERR_UNSUPPORTED for non-bf16 inputs or k_sel > 64.
 */
size_t nsa_selected_attn_bwd_workspace_size(int32_t batch, int32_t rows_total,
                                            int32_t max_seqlen_k, int32_t heads,
                                            int32_t kv_heads, int32_t k_sel);
size_t nsa_selected_attn_bwd_workspace_size_min(int32_t batch, int32_t rows_total,
                                                int32_t max_seqlen_k, int32_t heads,
                                                int32_t kv_heads, int32_t k_sel);
nsa_status nsa_selected_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                 const void* d_out, const float* lse, nsa_dtype dtype,
                                 const int32_t* indices, int32_t k_sel,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                                 int32_t heads, int32_t kv_heads, int32_t head_dim,
                                 int32_t block_size, float softmax_scale, float* dq, float* dk,
                                 float* dv, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Backward of the other two prefill branches and of the window mean.
 * [DeepSeek NSA with Triton, introduction and section 2.3 (the method is trained
 *  end to end, its kernels wrapped as a trainable module) and section 1.1 (the
 *  compressed branch over mean-pooled keys and values, the sliding-window
 *  branch).  The pages print no backward: these are the exact gradients of
 *  nsa_compressed_attn_fwd's output, nsa_window_attn_fwd's output and
 *  nsa_compress_k's means.]
 * Shared conventions: bf16 inputs, fp32 gradients, prefill rows (cu_seqlens_q
 * required; row r of sequence b at t = (r - cu_q[b]) + (L_b - Lq_b)).  `out` and
 * `lse` are the branch forward's output and natural-log normaliser, `d_out` the
 * upstream gradient of that output (for a gated sum, the gate times the
 * gradient of the sum: nsa_gates_bwd).  accumulate bit 0 clear: dq is written
 * in full, set: added to what dq holds; bit 1 likewise for the key and value
 * gradients (written in full means 0 for keys no row attends to).  With both
 * bits the branches of one step share dq, dk and dv.  Per head
 * over the row's keys J: dV_J += p dO^T; ds = p * (V_J dO - dO . out);
 * dq += scale ds K_J; dK_J += scale ds q^T.  Key gradients of a block seen by
 * more than 256 rows are summed with fp32 atomics (order may change between
 * calls: fp32 rounding only).  workspace: nsa_branch_attn_bwd_workspace_size
 * bytes (delta = dO . out per row and head).
 *
 * nsa_compressed_attn_bwd: keys are the compressed windows visible to t
 *   (stride*c + kernel - 1 <= t); k_c, v_c [N_c, kv_heads, 128] with
 *   cu_seqlens_c holding full-window counts; writes dq [rows, heads, 128] and
 *   dk_c, dv_c [N_c, kv_heads, 128].  Kernel 32, stride 16.
 * nsa_window_attn_bwd: keys max(0, t - window + 1) .. t; writes dq, dk, dv
 *   [N_k, kv_heads, 128].
 * nsa_gates_bwd: the gated sum o = g0 o_cmp + g1 o_sel + g2 o_win of
 *   nsa_prefill_step: d_out, o_cmp, o_sel, o_win [rows, heads, 128] bf16, gates
 *   [rows, heads, 3] float32 -> do_cmp, do_sel, do_win = g_b d_out (bf16,
 *   rounded to nearest even) and d_gates [rows, heads, 3] = d_out . o_b (fp32).
 * nsa_compress_bwd: the transpose of nsa_compress_k for fp32 gradients: dx[j]
 *   (+)= sum over the windows c holding token j of dx_c[c] / (valid tokens of
 *   window c); dx_c [N_c, heads, head_dim], dx [N, heads, head_dim], windows
 *   as in nsa_compress_k; tokens in no window get 0 (accumulate 0).
 */
size_t nsa_branch_attn_bwd_workspace_size(int32_t rows_total, int32_t heads);
nsa_status nsa_compressed_attn_bwd(const void* q, const void* k_c, const void* v_c,
                                   const void* o_cmp, const void* d_out, const float* lse,
                                   nsa_dtype dtype, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_c,
                                   int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                                   int32_t heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t kernel, int32_t stride, float softmax_scale,
                                   int32_t accumulate, float* dq, float* dk_c, float* dv_c,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
nsa_status nsa_window_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                               const void* d_out, const float* lse, nsa_dtype dtype,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                               int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t window,
                               float softmax_scale, int32_t accumulate, float* dq, float* dk,
                               float* dv, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);
nsa_status nsa_gates_bwd(const void* d_out, const void* o_cmp, const void* o_sel,
                         const void* o_win, nsa_dtype dtype, const float* gates, int32_t rows_total,
                         int32_t heads, int32_t head_dim, void* do_cmp, void* do_sel,
                         void* do_win, float* d_gates, hipStream_t stream);
nsa_status nsa_compress_bwd(const float* dx_c, float* dx, const int32_t* cu_seqlens,
                            const int32_t* cu_seqlens_c, int32_t batch, int32_t max_seqlen,
                            int32_t heads, int32_t head_dim, int32_t kernel, int32_t stride,
                            int32_t accumulate, hipStream_t stream);

/*
 * nsa_decode_step -- one decode step of the whole path for a packed batch: the
 * newest token of every sequence (t = L_b - 1) scores the compressed keys,
 * selects k blocks and attends to them.
 * [NOSA-1B core components, components 1-3 and the decode stage.]
 * With append_window != 0 the step first (re)computes the newest full window
 * (index n_c-1) of the K_c and pooled-CIS caches from the K and CIS caches, so a
 * caller that appended tokens completing a window gets an up-to-date cache.
 * Block choice: with n_cand == 0 one score per block, the compressed-attention
 * block score plus cis_weight times the block's pooled-CIS maximum (NOSA-1B
 * source analysis part 3, "beyond the kernel").  With n_cand > 0 the two-stage
 * choice of NOSA-1B core components, component 3: the n_cand best free blocks
 * by the compressed-attention score alone are the candidates, and the best
 * topk - |forced| of them by the pooled-CIS block maximum are kept (ties to the
 * lower id in both stages); needs cis_pooled; block_scores then receives the
 * compressed-attention scores alone.  The pages do not give n_cand.
 */
typedef struct nsa_decode_params {
  const void* q;            /* [batch, heads, head_dim], dtype */
  const void* k;            /* [N_k, kv_heads, head_dim], dtype */
  const void* v;            /* [N_k, kv_heads, head_dim], dtype */
  void* k_c;                /* [N_c, kv_heads, head_dim], kc_dtype (read; written if append) */
  const float* cis;         /* nullable [N_k, kv_heads]: importance scores */
  float* cis_pooled;        /* nullable [N_c, kv_heads] (read; written if append) */
  const int32_t* cu_seqlens_k; /* [batch+1] */
  const int32_t* cu_seqlens_c; /* [batch+1] full-window counts */
  void* out;                /* [batch, heads, head_dim], dtype (written) */
  float* block_scores;      /* nullable [batch, kv_heads, n_blocks_max] debug output */
  int32_t* indices;         /* nullable [batch, kv_heads, topk] debug output */
  nsa_dtype dtype;          /* q, k, v, out */
  nsa_dtype kc_dtype;       /* k_c */
  int32_t batch, max_seqlen_k, heads, kv_heads, head_dim;
  int32_t kernel, stride, block_size;
  int32_t topk, n_init, n_local;
  float cis_weight;         /* weight of the pooled CIS in the block score (needs cis_pooled) */
  int32_t cis_values;       /* != 0: CIS-scaled values with the ones normaliser (needs cis) */
  int32_t append_window;    /* != 0: refresh window n_c-1 of k_c / cis_pooled first */
  float softmax_scale;
  int32_t n_cand;           /* 0: one fused score; > 0: two-stage choice (needs cis_pooled) */
} nsa_decode_params;

size_t nsa_decode_workspace_size(const nsa_decode_params* p);
nsa_status nsa_decode_step(const nsa_decode_params* p, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * nsa_decode_step_noalloc -- nsa_decode_step for callers that cannot allocate
 * device memory (code under stream capture, serving loops and harnesses that
 * forbid allocation).  Same parameters, kernels and outputs as nsa_decode_step;
 * the workspace is a fixed device array inside the library instead of a caller
 * buffer: nsa_decode_noalloc_scratch_bytes() bytes (32 MiB) per GPU, held from
 * the library's load until the process ends.  Its device address is looked up
 * once per device on the first call there (the device of `stream`, or the
 * current one for the NULL stream).  The call allocates nothing.  Steps whose
 * workspace (nsa_decode_workspace_size) exceeds the scratch return
 * NSA_ERR_WORKSPACE before launching.  Every call on one GPU uses the same
 * scratch: calls that can overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  No part of the scratch
 * needs clearing between calls (the step writes every byte it reads).
 */
size_t nsa_decode_noalloc_scratch_bytes(void);
nsa_status nsa_decode_step_noalloc(const nsa_decode_params* p, hipStream_t stream);

/*
 * KV offload for decode: the K/V cache stays in host memory and each step moves
 * to the GPU only the selected blocks it does not already hold.
 * [NOSA-1B core components: the core idea (the whole KV cache offloaded to CPU
 *  memory, only the few important blocks brought back for each step's
 *  attention) and the decode stage.]
 * The caller owns the state, all of it in device memory:
 *   k_pool, v_pool  [batch*kv_heads, pool_slots, 64, head_dim] of the decode
 *                   dtype (nsa_offload_pool_bytes each): the K/V rows of the
 *                   blocks each (sequence, KV head) holds
 *   slot_of         int32 [batch*kv_heads, nb_cap]: the pool slot holding a
 *                   block, -1 if none
 *   block_of        int32 [batch*kv_heads, pool_slots]: the block a slot holds,
 *                   -1 if empty
 *   fetched         nullable int32 [batch*kv_heads], written by every step: the
 *                   blocks it copied from host memory
 * nsa_offload_reset marks every slot empty; call it before the first step and
 * whenever a (sequence, KV head) place of the batch changes owner.  Steps that
 * share a state must not overlap.  Limits: pool_slots <= 1024, nb_cap <= 4096.
 */
typedef struct nsa_offload_state {
  void* k_pool;
  void* v_pool;
  int32_t* slot_of;
  int32_t* block_of;
  int32_t* fetched;
  int32_t pool_slots;
  int32_t nb_cap;
} nsa_offload_state;
size_t nsa_offload_pool_bytes(int32_t batch, int32_t kv_heads, int32_t pool_slots,
                              int32_t head_dim, nsa_dtype dtype);
nsa_status nsa_offload_reset(const nsa_offload_state* o, int32_t batch, int32_t kv_heads,
                             hipStream_t stream);

/*
 * nsa_decode_step_offload -- nsa_decode_step with p->k and p->v in host memory
 * (pinned, hipHostMalloc), read by the GPU over the host link.  The step scores
 * and selects as nsa_decode_step does (compressed keys, CIS and every other
 * array stay in device memory; with append_window the newest window's 32 key
 * rows are read from host memory), then, per (sequence, KV head): listed
 * blocks already in a slot are kept; every other listed block takes the next
 * free slot (empty slots first, then slots holding a block this step does not
 * list, each in ascending order; misses in list order) and its 64 K and V rows
 * of that KV head are copied from host memory;
 * then attention runs over the pool.  The outputs equal nsa_decode_step's on
 * the same inputs.  bfloat16 only; topk <= 256 and topk <= pool_slots; blocks per
 * sequence <= nb_cap.  Errors as nsa_decode_step, plus NSA_ERR_INVALID_ARG /
 * NSA_ERR_UNSUPPORTED for a state outside these limits.
 *   workspace: nsa_decode_offload_workspace_size(p, o) bytes.
 */
size_t nsa_decode_offload_workspace_size(const nsa_decode_params* p, const nsa_offload_state* o);
nsa_status nsa_decode_step_offload(const nsa_decode_params* p, const nsa_offload_state* o,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nsa_compressed_attn_fwd -- compressed-branch attention of prefill rows, and
 * the block scores the selection reuses.
 * [DeepSeek NSA with Triton, section 1.1: the compressed branch attends to
 *  mean-pooled keys and values; the selected branch ranks blocks by the
 *  compressed-attention probabilities of the GQA group.]
 *   q            [rows, heads, head_dim] bfloat16 (prefill rows: cu_seqlens_q)
 *   k_c, v_c     [N_c, kv_heads, head_dim] bfloat16 (nsa_compress_k of K and V)
 *   o_cmp        [rows, heads, head_dim] of out_dtype (written): for query head h
 *                at position t, softmax over the windows visible to t of
 *                scale * q_h . k_c[c], times v_c; 0 when no window is visible
 *   lse          nullable [rows, heads] float32 (written): natural log of that
 *                softmax's normaliser, -inf when no window is visible
 *   block_scores nullable [rows, kv_heads, n_blocks_max] float32 (written): for
 *                block i, the max over the windows overlapping it of the group
 *                sum of the heads' probabilities; 0 past the row's windows and
 *                past the sequence's blocks
 *   workspace:   nsa_compressed_attn_workspace_size(...) bytes (the per-head
 *                normalisers and a transposed copy of v_c).
 *   bfloat16 only (the tiles run on the bf16 matrix cores); cu_seqlens_q is
 *   required.
 */
size_t nsa_compressed_attn_workspace_size(int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                                          int32_t heads, int32_t kv_heads, int32_t kernel,
                                          int32_t stride);
nsa_status nsa_compressed_attn_fwd(const void* q, const void* k_c, const void* v_c,
                                   nsa_dtype dtype, void* o_cmp, nsa_dtype out_dtype, float* lse,
                                   float* block_scores, int32_t n_blocks_max,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   const int32_t* cu_seqlens_c, int32_t batch, int32_t rows_total,
                                   int32_t max_seqlen_k, int32_t heads, int32_t kv_heads,
                                   int32_t head_dim, int32_t kernel, int32_t stride,
                                   int32_t block_size, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * nsa_blockmask_attn_fwd -- block-sparse attention driven by a block mask.
 * [TileLang NSA, section 1 (block-sparse attention): the attention matrix is
 *  cut into 64 x 64 blocks and a boolean block mask marks the ones computed;
 *  with is_causal the lower triangle only.]
 *   q, k, v  [N, heads, head_dim] bfloat16, packed by cu_seqlens [batch+1]
 *            (self-attention: query t of a sequence is its token t)
 *   mask     [batch, heads, nb, nb] uint8 (device), nb = ceil(max_seqlen / 64):
 *            nonzero at [b, h, i, j] = the queries of block i attend to the keys
 *            of block j
 *   causal   != 0: in addition, keys after the query's own position are ignored
 *            (blocks above the diagonal are skipped)
 *   out      [N, heads, head_dim] bfloat16 (written): softmax over the query's
 *            keys of scale * q.k, times v; 0 for a query with no key
 *   workspace: nsa_blockmask_attn_workspace_size(...) bytes (values transposed).
 *   bfloat16, head_dim 128, max_seqlen <= 32768; errors are reported before
 *   anything is launched.
 */
size_t nsa_blockmask_attn_workspace_size(int32_t batch, int32_t max_seqlen, int32_t heads);
nsa_status nsa_blockmask_attn_fwd(const void* q, const void* k, const void* v, nsa_dtype dtype,
                                  const uint8_t* mask, int32_t causal, void* out,
                                  const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                                  int32_t heads, int32_t head_dim, float softmax_scale,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nsa_window_attn_fwd -- sliding-window attention of prefill rows.
 * [DeepSeek NSA with Triton, section 1.1: the sliding-window branch attends to
 *  the most recent tokens, 512 in the pages' example.]
 *   Query position t attends to keys max(0, t - window + 1) .. t of its sequence
 *   (window keys including itself).  q [rows, heads, head_dim], k, v
 *   [N_k, kv_heads, head_dim], all bfloat16; out [rows, heads, head_dim] of
 *   out_dtype (written); lse nullable [rows, heads] float32 (natural log).
 *   workspace: nsa_window_attn_workspace_size(...) bytes (a transposed copy of v).
 */
size_t nsa_window_attn_workspace_size(int32_t batch, int32_t max_seqlen_k, int32_t kv_heads);
nsa_status nsa_window_attn_fwd(const void* q, const void* k, const void* v, nsa_dtype dtype,
                               void* out, nsa_dtype out_dtype, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                               int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t window,
                               float softmax_scale, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * nsa_prefill_step -- the three-branch NSA prefill of packed query rows.
 * [DeepSeek NSA with Triton, section 1.1: o = g_cmp * o_cmp + g_sel * o_sel +
 *  g_win * o_win, gates per token and head; selection from the compressed
 *  probabilities of the group; TileLang NSA, section 2, for the selected blocks.]
 * Steps: mean-pool K and V into k_c, v_c (written); compressed attention with
 * block scores; top-`topk` blocks per (row, kv head) with n_init / n_local forced
 * blocks (0 and 0 for the pages' configuration); attention over the selected
 * blocks; sliding-window attention; the gated sum into out.  The compressed and
 * selected branch outputs wait in the workspace as bfloat16 rows (fp32
 * accumulation inside each branch); the gated sum is formed in fp32 and
 * rounded once.  bfloat16 only.
 */
typedef struct nsa_prefill_params {
  const void* q;               /* [rows, heads, head_dim] bf16 */
  const void* k;               /* [N_k, kv_heads, head_dim] bf16 */
  const void* v;               /* [N_k, kv_heads, head_dim] bf16 */
  void* k_c;                   /* [N_c, kv_heads, head_dim] bf16 (written) */
  void* v_c;                   /* [N_c, kv_heads, head_dim] bf16 (written) */
  const float* gates;          /* [rows, heads, 3]: compressed, selected, window */
  const int32_t* cu_seqlens_q; /* [batch+1] */
  const int32_t* cu_seqlens_k; /* [batch+1] */
  const int32_t* cu_seqlens_c; /* [batch+1] full-window counts */
  void* out;                   /* [rows, heads, head_dim] bf16 (written) */
  float* block_scores;         /* nullable [rows, kv_heads, n_blocks_max] debug output */
  int32_t* indices;            /* nullable [rows, kv_heads, topk] debug output */
  nsa_dtype dtype;             /* must be NSA_BF16 */
  int32_t batch, rows_total, max_seqlen_k, heads, kv_heads, head_dim;
  int32_t kernel, stride, block_size;
  int32_t topk, n_init, n_local, window;
  float softmax_scale;
} nsa_prefill_params;

/*
 * Workspace: nsa_prefill_workspace_size(p) bytes (16-byte aligned) run the
 * selected branch key-block stationary (as nsa_selected_attn_fwd given a
 * workspace; the size includes its partial states, rows * heads * topk * 264
 * bytes, its block lists, rows * kv_heads * topk * 10 bytes, and its merged
 * rows in float32 until the gated sum, rows * heads * 512 bytes); any size
 * from nsa_prefill_workspace_size_min(p) up to that, or more than 8192 blocks
 * per sequence, runs it row by row.  Less: NSA_ERR_WORKSPACE.
 */
size_t nsa_prefill_workspace_size(const nsa_prefill_params* p);
size_t nsa_prefill_workspace_size_min(const nsa_prefill_params* p);
nsa_status nsa_prefill_step(const nsa_prefill_params* p, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
