// Internal launchers behind the C ABI (host side).  Arguments are validated by
// the API layer before any of these is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

struct bf16_t;

// Window geometry the scoring kernels are compiled for.
constexpr int kKernel = 32;
constexpr int kStride = 16;
constexpr int kBlock = 64;
constexpr int kHeadDim = 128;
constexpr float kLog2eHost = 1.4426950408889634f;

// Windows per workgroup of the logits kernel; blocks per workgroup of the
// block-score kernel; the largest per-row block count the top-k sort holds.
constexpr int kChunkWindows = 64;
constexpr int kBlocksPerWG = 256;
constexpr int kMaxSortBlocks = 4096;
// Partial states one decode (row, kv head) may be split into.
constexpr int kMaxSplits = 64;
// The decode kernel that selects and attends in one launch handles sequences of
// up to this many blocks and up to this many selected blocks; batches whose
// longest sequence has at most kFusedSmallBlocks blocks use a lighter variant.
constexpr int kFusedMaxBlocks = 2048;
constexpr int kFusedMidBlocks = 1024;
constexpr int kFusedSmallBlocks = 512;
constexpr int kFusedMaxSel = 256;
// KV offload: block slots per (sequence, KV head) in the device pool, and the
// largest top-k the offloaded decode step handles (one plan thread per place).
constexpr int kMaxPoolSlots = 1024;
constexpr int kMaxOffloadSel = 256;

// Kernel kinds that a profiling request can target.
enum KernelKind {
  kKindPool = 0,
  kKindLogits = 1,
  kKindBlockScores = 2,
  kKindAttn = 3,
  kKindCombine = 4,
  kKindCmpLse = 5,
  kKindCmpProbs = 6,
  kKindWindow = 7,
  kKindFetch = 8,
  kKindMask = 9,
  kKindBwdQ = 10,     // selected-attention backward: dq
  kKindBwdKV = 11,    // selected-attention backward: dk and dv
  kKindBwdLists = 12, // selected-attention backward: delta and the per-block row lists
  kKindBwdQMerge = 13, // selected-attention backward, key-block dq: the sum of its partial states
  kKindBlockLists = 14, // key-block selected attention: the per-chunk block lists
  kKindCount = 15
};

// One armed (start, stop) event pair per kernel kind, per host thread.
struct ProfSlot {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool armed = false;
};
ProfSlot& prof_slot(int kind);

// Launch `kernel`; if a profiling request is armed for `kind`, the launch records
// its events at the kernel's own start and end (hipExtLaunchKernelGGL) and the
// request is consumed.
template <typename Kernel, typename... Args>
hipError_t launch_kernel(int kind, Kernel kernel, dim3 grid, dim3 block, hipStream_t s,
                         Args... args) {
  ProfSlot& p = prof_slot(kind);
  if (p.armed) {
    p.armed = false;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, p.start, p.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
  return hipGetLastError();
}

hipError_t launch_mean_pool(const void* x, int x_bf16, void* y, int y_bf16, const int* cu,
                            const int* cuc, int batch, int max_windows, int width, int kernel,
                            int stride, int last_n, hipStream_t s);

// Scoring workspace carve-up (decode rows).
struct ScoresWs {
  float* logits;  // [batch, kv_heads, G, n_chunk_max*64] exp2(logit - chunk max), log2 domain
  float2* part;   // [batch, kv_heads, n_chunk_max, G] chunk (max, sum of exp2)
  float* cisb;    // [batch, kv_heads, n_chunk_max*16+1] per-block CIS maxima
};
size_t scores_ws_bytes(int batch, int kv_heads, int group, int max_seqlen_k);
// Layout of the scoring workspace for sequences of up to max_seqlen_k tokens.
struct ScoreDims {
  int nc_max, nb_max, n_chunk_max, ldc, ldb;
};
ScoreDims score_dims(int max_seqlen_k);
ScoresWs scores_ws_carve(void* base, int batch, int kv_heads, int group, int max_seqlen_k);

struct DecodeScoresArgs {
  const void* q;
  int q_bf16;
  void* kc;  // compressed keys; its newest window is rewritten when refresh_k is set
  int kc_bf16;
  float* cis_pooled;  // nullable: fused with cis_weight; newest window rewritten with refresh_cis
  float cis_weight;
  float* block_scores;  // nullable output
  float* window_probs;  // nullable output
  const int* cu_k;
  const int* cu_c;
  int batch, max_seqlen_k, heads, kv_heads;
  float scale_log2;
  ScoresWs ws;
  int* indices;  // nullable: no selection
  int topk, n_init, n_local;
  int n_cand;                  // > 0: two-stage selection (candidates, then CIS re-rank)
  const void* refresh_k;       // nullable: recompute the newest window from these keys
  const float* refresh_cis;    // nullable: and the newest pooled CIS from these scores
  int logits_only;             // launch the logits kernel only (the selection runs elsewhere)
};
hipError_t launch_decode_scores(const DecodeScoresArgs& a, hipStream_t s);

hipError_t launch_select_topk(const float* block_scores, int* indices, const int* cu_q,
                              const int* cu_k, int batch, int rows_total, int kv_heads,
                              int nb_max, int topk, int n_init, int n_local, hipStream_t s);

// Attention workspace carve-up.
struct AttnWs {
  float2* part_ml;  // [units, n_split, G] (max, sum) per split
  float* part_acc;  // [units, n_split, G, D]
};
int attn_split_blocks(int batch, int kv_heads, int k_sel);  // selected blocks per workgroup
size_t attn_ws_bytes(int rows_total, int kv_heads, int group, int k_sel, int decode);
AttnWs attn_ws_carve(void* base, int rows_total, int kv_heads, int group, int k_sel, int decode);

// out_f32: prefill rows only (bf16 inputs): write float32 rows there instead of out.
hipError_t launch_selected_attn(const void* q, const void* k, const void* v, int bf16,
                                const int* indices, int k_sel, const float* cis, void* out,
                                float* lse, const int* cu_q, const int* cu_k, int batch,
                                int rows_total, int heads, int kv_heads, float scale_log2,
                                const AttnWs& ws, hipStream_t s, float* out_f32 = nullptr);

// Prefill rows, key-block stationary (bf16): partial states per (row, head,
// place) in `ws` (block_attn_ws_bytes), then their merge.  Writes out (bf16) or
// out_f32 when given, and lse when given.  block_attn_grid_fits: the launch
// shapes stay within the grid limits and the 32-bit offsets of the kernels.
size_t block_attn_ws_bytes(int rows_total, int heads, int kv_heads, int k_sel);
bool block_attn_grid_fits(int batch, int rows_total, int heads, int kv_heads, int max_seqlen_k,
                          int k_sel);
hipError_t launch_block_attn(const void* q, const void* k, const void* v, const int* indices,
                             int k_sel, const float* cis, void* out, float* out_f32, float* lse,
                             const int* cu_q, const int* cu_k, int batch, int rows_total,
                             int heads, int kv_heads, int max_seqlen_k, float scale_log2,
                             void* ws, hipStream_t s);

// Decode: selection and attention in one launch (bf16; nb_max <= kFusedMaxBlocks,
// topk <= kFusedMaxSel), after the logits kernel, then the merge of the splits.
hipError_t launch_select_attn(const DecodeScoresArgs& a, const void* k, const void* v,
                              const float* cis_values, void* out, const AttnWs& ws,
                              hipStream_t s);

// KV offload (decode): plan the fetches of the listed blocks that are not in the
// pool, copy them from the caller's K/V (host memory), attend over the pool.
struct OffloadArgs {
  const int* indices;    // [units, k_sel] listed blocks, ascending, -1 padded
  int k_sel, units, kv_heads, nb_cap, pool_slots;
  int* slot_of;          // [units, nb_cap]: slot of a resident block, else -1
  int* block_of;         // [units, pool_slots]: block held by a slot, else -1
  int* slot_ids;         // [units, k_sel] workspace: slot of each listed block
  int2* copies;          // [units, k_sel] workspace: (block, slot) of each miss
  int* n_copy;           // [units] workspace: misses
  int* fetched;          // nullable [units]: misses, for the caller
  const bf16_t* k_src;   // [N_k, kv_heads, 128] (host memory)
  const bf16_t* v_src;
  const int* cu_k;
  bf16_t* kpool;         // [units, pool_slots, 64, 128]
  bf16_t* vpool;
};
hipError_t launch_offload_reset(int* slot_of, size_t n_slot_of, int* block_of, size_t n_block_of,
                                hipStream_t s);
hipError_t launch_offload_fetch(const OffloadArgs& a, hipStream_t s);
hipError_t launch_pool_attn(const void* q, const OffloadArgs& a, const float* cis_values,
                            void* out, int heads, float scale_log2, const AttnWs& ws,
                            hipStream_t s);

// Prefill branches (bf16, prefill rows).
struct CompressedPrefillArgs {
  const bf16_t* q;
  const bf16_t* kc;
  const bf16_t* vc;
  const int* cu_q;
  const int* cu_k;
  const int* cu_c;
  int batch, rows_total, max_seqlen_q, max_windows, heads, kv_heads;
  float scale_log2;
  float* lse2;           // [rows, heads] workspace: log2-domain normaliser
  bf16_t* vct;           // workspace: v_c transposed, transposed_bytes(batch, kv, max_windows)
  void* o_cmp;           // [rows, heads, 128]
  int out_f32;           // o_cmp dtype: 1 float32, 0 bfloat16
  float* lse_nat;        // nullable [rows, heads]
  float* block_scores;   // nullable [rows, kv_heads, nb_max]
  int nb_max;
};
hipError_t launch_compressed_prefill(const CompressedPrefillArgs& a, hipStream_t s);

struct WindowPrefillArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const int* cu_q;
  const int* cu_k;
  int batch, rows_total, max_seqlen_q, max_seqlen_k, heads, kv_heads, window;
  float scale_log2;
  bf16_t* vt;            // workspace: v transposed, transposed_bytes(batch, kv, max_seqlen_k)
  void* out;
  int out_f32;
  float* lse_nat;        // nullable
  const float* gates;    // nullable [rows, heads, 3]: gated sum with o_cmp and o_sel
  const bf16_t* o_cmp;   // [rows, heads, 128] (with gates)
  const bf16_t* o_sel;   // [rows, heads, 128] (with gates)
  const float* o_sel32;  // nullable [rows, heads, 128]: o_sel as float32 rows instead
};
hipError_t launch_window_prefill(const WindowPrefillArgs& a, hipStream_t s);

// Block-mask attention (multi-head, bf16): longest sequence it takes.
constexpr int kBlockMaskMaxLen = 32768;
hipError_t launch_blockmask_attn(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                 const unsigned char* mask, int causal, bf16_t* out,
                                 const int* cu, int batch, int max_seqlen, int heads,
                                 float scale_log2, bf16_t* vt, hipStream_t s);

// Backward of an attention branch over prefill rows (bf16 inputs, fp32
// gradients).  The keys of a row are the tokens of its listed blocks (selected
// branch), the last `window` tokens (sliding-window branch) or the compressed
// windows visible to it (compressed branch; k, v are then K_c, V_c).
enum BwdMode { kBwdSelected = 0, kBwdWindow = 1, kBwdCompressed = 2 };
struct SelectedBwdArgs {
  int mode;            // BwdMode
  int window;          // kBwdWindow: keys t - window + 1 .. t
  int accumulate;      // bit 0: add to dq; bit 1: add to dk, dv (instead of writing)
  const int* cu_kv;    // key rows of each sequence (cu_k, or cu_c for compressed keys)
  const bf16_t* q;     // [rows, heads, 128]
  const bf16_t* k;     // [N_kv, kv_heads, 128]
  const bf16_t* v;
  const bf16_t* out;   // [rows, heads, 128] forward output
  const bf16_t* dout;  // [rows, heads, 128] its upstream gradient
  const float* lse;    // [rows, heads] forward natural-log normaliser
  const int* indices;  // [rows, kv_heads, k_sel]
  int k_sel;
  const int* cu_q;
  const int* cu_k;
  int batch, rows_total, heads, kv_heads, nb_max, max_seqlen_k;  // nb_max: key blocks
  float scale;         // softmax scale (natural domain)
  float* dq;           // [rows, heads, 128]
  float* dk;           // [N_k, kv_heads, 128]
  float* dv;
  // workspace (selected_bwd_ws_carve)
  float* delta;        // [rows, heads]
  int* cnt;            // [batch, kv_heads, nb_max] rows listing each block
  int* off;            // list offsets
  int* cursor;         // fill cursors
  int2* list;          // [rows * kv_heads * k_sel] (row, position), grouped by block
  bf16_t* dq_part;     // nullable: the key-block dq's partial states (block_dq_ws_bytes);
                       // without it dq runs one workgroup per (row, KV head)
};
size_t selected_bwd_ws_bytes(int rows_total, int heads, int kv_heads, int k_sel, int batch,
                             int nb_max);
void selected_bwd_ws_carve(void* base, SelectedBwdArgs& a);
hipError_t launch_selected_bwd(const SelectedBwdArgs& a, hipStream_t s);
// Selected-attention dq, key-block stationary (attn_blocks.hip): partial dq per
// (row, place, head) in a.dq_part, then their sum into a.dq.
size_t block_dq_ws_bytes(int rows_total, int heads, int kv_heads, int k_sel);
hipError_t launch_block_dq(const SelectedBwdArgs& a, hipStream_t s);
// The matrix-core kernels: dk/dv of every key set, dq of the window and
// compressed key sets (bwd_mfma.hip).
hipError_t launch_bwd_mfma(const SelectedBwdArgs& a, hipStream_t s);
int mfma_bwd_rows_per_chunk(int mode);  // rows of a block one dk/dv workgroup takes
hipError_t launch_gates_bwd(const bf16_t* dout, const bf16_t* o_cmp, const bf16_t* o_sel,
                            const bf16_t* o_win, const float* gates, size_t n_rh, bf16_t* do_cmp,
                            bf16_t* do_sel, bf16_t* do_win, float* d_gates, hipStream_t s);
// dx[j] (+)= sum over the windows c holding token j of dx_c[c] / (valid tokens of c)
hipError_t launch_pool_bwd(const float* dxc, float* dx, const int* cu, const int* cu_c, int batch,
                           int n_tokens_max, int width, int kernel, int stride, int accumulate,
                           hipStream_t s);

// Values transposed per (sequence, KV head, dim) for the prefill branches.
int transposed_ld(int max_len);
size_t transposed_bytes(int batch, int kv_heads, int max_len);

}  // namespace nsa
