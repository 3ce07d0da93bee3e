// Host side of the C ABI declared in include/nsa.h: argument validation, grid
// sizing, workspace carve-up and kernel launches on the caller's stream.  No
// allocation, no synchronisation.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/nsa.h"
#include "checks.h"
#include "launch.h"

namespace {

thread_local std::string g_err;
thread_local nsa::ProfSlot g_prof[nsa::kKindCount];

nsa_status fail(nsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

nsa_status ok() {
  g_err.clear();
  return NSA_OK;
}

nsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int d) { return d == NSA_F32 || d == NSA_BF16; }
bool group_ok(int heads, int kv_heads) {
  if (kv_heads <= 0 || heads <= 0 || heads % kv_heads) return false;
  const int g = heads / kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}
// Selected blocks per row: a prefill workgroup stages all of its row's ids at
// once; decode splits a row over at most kMaxSplits workgroups.
constexpr int kMaxPrefillSel = 64;
constexpr int kMaxDecodeSel = 64 * nsa::kMaxSplits;

float scale_log2_of(float softmax_scale, int head_dim) {
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(head_dim));
  return sc * nsa::kLog2eHost;
}

// Debug mode: run the device checks `body` adds to `chk` and fail the call,
// before any of its work is launched, when one finds a broken precondition.
#define NSA_DEVICE_CHECKS(fn, stream, body)                                      \
  do {                                                                           \
    if (nsa::debug_checks_on()) {                                                \
      nsa::DebugChecks chk(stream);                                              \
      body;                                                                      \
      char msg_[256];                                                            \
      if (chk.failed(msg_, sizeof(msg_))) return fail(NSA_ERR_INVALID_ARG, "%s: %s", fn, msg_); \
    }                                                                            \
  } while (0)

#define NSA_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

nsa_status check_geometry(const char* fn, int head_dim, int kernel, int stride, int block) {
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  NSA_REQUIRE(kernel == nsa::kKernel && stride == nsa::kStride, NSA_ERR_UNSUPPORTED,
              "%s: window %d/stride %d unsupported (32/16 only)", fn, kernel, stride);
  NSA_REQUIRE(block == nsa::kBlock, NSA_ERR_UNSUPPORTED, "%s: block_size %d unsupported (64 only)", fn, block);
  return NSA_OK;
}

}  // namespace

nsa::ProfSlot& nsa::prof_slot(int kind) { return g_prof[kind]; }

namespace nsa {
// The nsa_last_error text for entry points defined in other sources.
nsa_status set_error(nsa_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace nsa

extern "C" {

const char* nsa_last_error(void) { return g_err.c_str(); }

nsa_status nsa_profile_next_launch(int32_t kernel_kind, hipEvent_t start, hipEvent_t stop) {
  NSA_REQUIRE(kernel_kind >= 0 && kernel_kind < nsa::kKindCount, NSA_ERR_INVALID_ARG,
              "nsa_profile_next_launch: unknown kernel kind %d", kernel_kind);
  NSA_REQUIRE(start != nullptr && stop != nullptr, NSA_ERR_INVALID_ARG,
              "nsa_profile_next_launch: null event");
  nsa::ProfSlot& p = g_prof[kernel_kind];
  p.start = start;
  p.stop = stop;
  p.armed = true;
  return ok();
}

int32_t nsa_version(void) { return 200; }

int32_t nsa_set_debug_checks(int32_t on) { return nsa::set_debug_checks(on); }

int32_t nsa_window_count(int32_t length, int32_t kernel, int32_t stride, int32_t tail_mode) {
  if (length < 0 || kernel < 1 || stride < 1 || (tail_mode != 0 && tail_mode != 1)) return -1;
  if (length == 0) return 0;
  if (tail_mode == 0) return length >= kernel ? (length - kernel) / stride + 1 : 0;
  if (length <= kernel) return 1;
  return (length - kernel + stride - 1) / stride + 1;
}

nsa_status nsa_compress_k(const void* x, nsa_dtype x_dtype, void* x_c, nsa_dtype xc_dtype,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_c, int32_t batch,
                          int32_t max_windows, int32_t heads, int32_t head_dim, int32_t kernel,
                          int32_t stride, hipStream_t stream) {
  NSA_REQUIRE(batch >= 0 && max_windows >= 0, NSA_ERR_INVALID_ARG, "nsa_compress_k: negative batch or max_windows");
  NSA_REQUIRE(heads > 0 && head_dim > 0, NSA_ERR_INVALID_ARG, "nsa_compress_k: heads and head_dim must be positive");
  NSA_REQUIRE(kernel >= 1 && stride >= 1, NSA_ERR_INVALID_ARG, "nsa_compress_k: kernel and stride must be >= 1");
  NSA_REQUIRE(dtype_ok(x_dtype) && dtype_ok(xc_dtype), NSA_ERR_UNSUPPORTED, "nsa_compress_k: unknown dtype");
  if (batch == 0 || max_windows == 0) return ok();
  NSA_REQUIRE(x && x_c && cu_seqlens && cu_seqlens_c, NSA_ERR_INVALID_ARG, "nsa_compress_k: null pointer");
  NSA_REQUIRE(aligned16(x) && aligned16(x_c), NSA_ERR_INVALID_ARG, "nsa_compress_k: tensors must be 16-byte aligned");
  const long width = long(heads) * head_dim;
  NSA_REQUIRE(width < (1L << 30), NSA_ERR_INVALID_ARG, "nsa_compress_k: row too wide");
  NSA_DEVICE_CHECKS("nsa_compress_k", stream, {
    chk.cu(cu_seqlens, batch, -1, nsa::kCheckCuK);
    chk.cu(cu_seqlens_c, batch, max_windows, nsa::kCheckCuC);
    chk.windows(cu_seqlens, cu_seqlens_c, batch, kernel, stride);
  });
  return hip_status(nsa::launch_mean_pool(x, x_dtype == NSA_BF16, x_c, xc_dtype == NSA_BF16,
                                          cu_seqlens, cu_seqlens_c, batch, max_windows,
                                          int(width), kernel, stride, 0, stream),
                    "nsa_compress_k");
}

nsa_status nsa_cis_mean_pool_varlen(const float* cis, float* cis_pooled, const int32_t* cu_seqlens,
                                    const int32_t* cu_seqlens_c, int32_t batch,
                                    int32_t max_windows, int32_t heads, int32_t kernel,
                                    int32_t stride, hipStream_t stream) {
  NSA_REQUIRE(batch >= 0 && max_windows >= 0, NSA_ERR_INVALID_ARG, "nsa_cis_mean_pool_varlen: negative batch or max_windows");
  NSA_REQUIRE(heads > 0, NSA_ERR_INVALID_ARG, "nsa_cis_mean_pool_varlen: heads must be positive");
  NSA_REQUIRE(kernel >= 1 && stride >= 1, NSA_ERR_INVALID_ARG, "nsa_cis_mean_pool_varlen: kernel and stride must be >= 1");
  if (batch == 0 || max_windows == 0) return ok();
  NSA_REQUIRE(cis && cis_pooled && cu_seqlens && cu_seqlens_c, NSA_ERR_INVALID_ARG, "nsa_cis_mean_pool_varlen: null pointer");
  NSA_DEVICE_CHECKS("nsa_cis_mean_pool_varlen", stream, {
    chk.cu(cu_seqlens, batch, -1, nsa::kCheckCuK);
    chk.cu(cu_seqlens_c, batch, max_windows, nsa::kCheckCuC);
    chk.windows(cu_seqlens, cu_seqlens_c, batch, kernel, stride);
  });
  return hip_status(nsa::launch_mean_pool(cis, 0, cis_pooled, 0, cu_seqlens, cu_seqlens_c, batch,
                                          max_windows, heads, kernel, stride, 0, stream),
                    "nsa_cis_mean_pool_varlen");
}

size_t nsa_compressed_scores_workspace_size(int32_t batch, int32_t max_seqlen_k, int32_t heads,
                                            int32_t kv_heads, int32_t kernel, int32_t stride) {
  if (batch <= 0 || kv_heads <= 0 || heads <= 0 || kernel < 1 || stride < 1) return 0;
  return nsa::scores_ws_bytes(batch, kv_heads, heads / kv_heads, max_seqlen_k);
}

nsa_status nsa_compressed_scores(const void* q, nsa_dtype q_dtype, const void* k_c,
                                 nsa_dtype kc_dtype, const float* cis_pooled, float cis_weight,
                                 float* block_scores, float* window_probs,
                                 const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_c,
                                 int32_t batch, int32_t max_seqlen_k, int32_t heads,
                                 int32_t kv_heads, int32_t head_dim, int32_t kernel,
                                 int32_t stride, int32_t block_size, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_compressed_scores";
  NSA_REQUIRE(batch >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: negative batch or max_seqlen_k", fn);
  NSA_REQUIRE(group_ok(heads, kv_heads), NSA_ERR_UNSUPPORTED, "%s: heads %d / kv_heads %d unsupported", fn, heads, kv_heads);
  NSA_REQUIRE(dtype_ok(q_dtype) && dtype_ok(kc_dtype), NSA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  nsa_status st = check_geometry(fn, head_dim, kernel, stride, block_size);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(std::isfinite(cis_weight), NSA_ERR_INVALID_ARG, "%s: cis_weight must be finite", fn);
  NSA_REQUIRE((max_seqlen_k + block_size - 1) / block_size <= nsa::kMaxSortBlocks, NSA_ERR_UNSUPPORTED,
              "%s: more than %d blocks per sequence", fn, nsa::kMaxSortBlocks);
  if (batch == 0) return ok();
  NSA_REQUIRE(q && k_c && block_scores && cu_seqlens_k && cu_seqlens_c, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k_c), NSA_ERR_INVALID_ARG, "%s: q and k_c must be 16-byte aligned", fn);
  const size_t need = nsa_compressed_scores_workspace_size(batch, max_seqlen_k, heads, kv_heads, kernel, stride);
  NSA_REQUIRE(workspace != nullptr || need == 0, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  nsa::DecodeScoresArgs a{};
  a.q = q;
  a.q_bf16 = q_dtype == NSA_BF16;
  a.kc = const_cast<void*>(k_c);
  a.kc_bf16 = kc_dtype == NSA_BF16;
  a.cis_pooled = const_cast<float*>(cis_pooled);  // read only: no refresh here
  a.cis_weight = cis_weight;
  a.block_scores = block_scores;
  a.window_probs = window_probs;
  a.cu_k = cu_seqlens_k;
  a.cu_c = cu_seqlens_c;
  a.batch = batch;
  a.max_seqlen_k = max_seqlen_k;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.scale_log2 = scale_log2_of(softmax_scale, head_dim);
  a.ws = nsa::scores_ws_carve(workspace, batch, kv_heads, heads / kv_heads, max_seqlen_k);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_seqlens_c, batch, -1, nsa::kCheckCuC);
    chk.windows(cu_seqlens_k, cu_seqlens_c, batch, kernel, stride);
  });
  return hip_status(nsa::launch_decode_scores(a, stream), fn);
}

nsa_status nsa_select_topk(const float* block_scores, int32_t* indices, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int32_t batch, int32_t rows_total,
                           int32_t max_seqlen_k, int32_t kv_heads, int32_t n_blocks_max, int32_t k,
                           int32_t n_init, int32_t n_local, int32_t block_size, hipStream_t stream) {
  const char* fn = "nsa_select_topk";
  NSA_REQUIRE(batch >= 0 && rows_total >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(kv_heads > 0, NSA_ERR_INVALID_ARG, "%s: kv_heads must be positive", fn);
  NSA_REQUIRE(block_size == nsa::kBlock, NSA_ERR_UNSUPPORTED, "%s: block_size %d unsupported (64 only)", fn, block_size);
  NSA_REQUIRE(k >= 1, NSA_ERR_INVALID_ARG, "%s: k must be >= 1", fn);
  NSA_REQUIRE(n_init >= 0 && n_local >= 0 && n_init + n_local <= k, NSA_ERR_INVALID_ARG,
              "%s: need 0 <= n_init, 0 <= n_local, n_init + n_local <= k", fn);
  NSA_REQUIRE(n_blocks_max >= (max_seqlen_k + block_size - 1) / block_size, NSA_ERR_INVALID_ARG,
              "%s: n_blocks_max %d < ceil(max_seqlen_k / block_size)", fn, n_blocks_max);
  NSA_REQUIRE(n_blocks_max <= nsa::kMaxSortBlocks, NSA_ERR_UNSUPPORTED,
              "%s: %d blocks per row exceed the supported %d", fn, n_blocks_max, nsa::kMaxSortBlocks);
  if (cu_seqlens_q == nullptr)
    NSA_REQUIRE(rows_total == batch, NSA_ERR_INVALID_ARG, "%s: decode needs rows_total == batch", fn);
  if (rows_total == 0 || batch == 0) return ok();
  NSA_REQUIRE(block_scores && indices && cu_seqlens_k, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_seqlens_q, batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(cu_seqlens_q, cu_seqlens_k, batch);
    chk.no_nan(block_scores, long(rows_total) * kv_heads * n_blocks_max);
  });
  return hip_status(nsa::launch_select_topk(block_scores, indices, cu_seqlens_q, cu_seqlens_k, batch,
                                            rows_total, kv_heads, n_blocks_max, k, n_init, n_local,
                                            stream),
                    fn);
}

size_t nsa_selected_attn_workspace_size(int32_t rows_total, int32_t heads, int32_t kv_heads,
                                        int32_t head_dim, int32_t k_sel, int32_t decode) {
  if (rows_total <= 0 || kv_heads <= 0 || heads <= 0 || k_sel <= 0 || head_dim != nsa::kHeadDim) return 0;
  if (!decode) return k_sel <= kMaxPrefillSel ? nsa::block_attn_ws_bytes(rows_total, heads, kv_heads, k_sel) : 0;
  return nsa::attn_ws_bytes(rows_total, kv_heads, heads / kv_heads, k_sel, decode);
}

nsa_status nsa_selected_attn_fwd(const void* q, const void* k, const void* v, nsa_dtype dtype,
                                 const int32_t* indices, int32_t k_sel, const float* cis,
                                 void* out, float* lse, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t batch, int32_t rows_total,
                                 int32_t max_seqlen_k, int32_t heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t block_size, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_selected_attn_fwd";
  NSA_REQUIRE(batch >= 0 && rows_total >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(dtype_ok(dtype), NSA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  NSA_REQUIRE(group_ok(heads, kv_heads), NSA_ERR_UNSUPPORTED, "%s: heads %d / kv_heads %d unsupported", fn, heads, kv_heads);
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  NSA_REQUIRE(block_size == nsa::kBlock, NSA_ERR_UNSUPPORTED, "%s: block_size %d unsupported (64 only)", fn, block_size);
  NSA_REQUIRE(k_sel >= 1, NSA_ERR_INVALID_ARG, "%s: k_sel must be >= 1", fn);
  const int decode = cu_seqlens_q == nullptr;
  NSA_REQUIRE(k_sel <= (decode ? kMaxDecodeSel : kMaxPrefillSel), NSA_ERR_UNSUPPORTED,
              "%s: k_sel %d above the supported %d", fn, k_sel, decode ? kMaxDecodeSel : kMaxPrefillSel);
  if (decode)
    NSA_REQUIRE(rows_total == batch, NSA_ERR_INVALID_ARG, "%s: decode needs rows_total == batch", fn);
  NSA_REQUIRE(!decode || rows_total <= 65535, NSA_ERR_UNSUPPORTED, "%s: decode batch above 65535", fn);
  if (rows_total == 0 || batch == 0) return ok();
  NSA_REQUIRE(q && k && v && indices && out && cu_seqlens_k, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), NSA_ERR_INVALID_ARG,
              "%s: q, k, v, out must be 16-byte aligned", fn);
  const size_t need = nsa_selected_attn_workspace_size(rows_total, heads, kv_heads, head_dim, k_sel, decode);
  // prefill rows: the workspace is optional (none, or float32 inputs: the
  // row-by-row kernel)
  const bool blocks = !decode && workspace_bytes > 0 && dtype == NSA_BF16;
  if (decode || blocks) {
    NSA_REQUIRE(workspace != nullptr || need == 0, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
    NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  }
  if (blocks) {
    NSA_REQUIRE(aligned16(workspace), NSA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
    NSA_REQUIRE(nsa::block_attn_grid_fits(batch, rows_total, heads, kv_heads, max_seqlen_k, k_sel), NSA_ERR_UNSUPPORTED,
                "%s: shape too large for the key-block path", fn);
  }
  const nsa::AttnWs ws = nsa::attn_ws_carve(workspace, rows_total, kv_heads, heads / kv_heads, k_sel, decode);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_seqlens_q, batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(cu_seqlens_q, cu_seqlens_k, batch);
    chk.unique_ids(indices, long(rows_total) * kv_heads, k_sel);
  });
  if (blocks)
    return hip_status(nsa::launch_block_attn(q, k, v, indices, k_sel, cis, out, nullptr, lse,
                                             cu_seqlens_q, cu_seqlens_k, batch, rows_total, heads,
                                             kv_heads, max_seqlen_k,
                                             scale_log2_of(softmax_scale, head_dim), workspace,
                                             stream),
                      fn);
  return hip_status(nsa::launch_selected_attn(q, k, v, dtype == NSA_BF16, indices, k_sel, cis, out,
                                              lse, cu_seqlens_q, cu_seqlens_k, batch, rows_total,
                                              heads, kv_heads, scale_log2_of(softmax_scale, head_dim),
                                              ws, stream),
                    fn);
}

size_t nsa_selected_attn_bwd_workspace_size(int32_t batch, int32_t rows_total,
                                            int32_t max_seqlen_k, int32_t heads,
                                            int32_t kv_heads, int32_t k_sel) {
  if (batch <= 0 || rows_total <= 0 || max_seqlen_k <= 0 || heads <= 0 || kv_heads <= 0 ||
      k_sel <= 0)
    return 0;
  const int nb_max = (max_seqlen_k + nsa::kBlock - 1) / nsa::kBlock;
  return ((nsa::selected_bwd_ws_bytes(rows_total, heads, kv_heads, k_sel, batch, nb_max) + 255) & ~size_t(255)) +
         nsa::block_dq_ws_bytes(rows_total, heads, kv_heads, k_sel);
}

size_t nsa_selected_attn_bwd_workspace_size_min(int32_t batch, int32_t rows_total,
                                                int32_t max_seqlen_k, int32_t heads,
                                                int32_t kv_heads, int32_t k_sel) {
  if (batch <= 0 || rows_total <= 0 || max_seqlen_k <= 0 || heads <= 0 || kv_heads <= 0 ||
      k_sel <= 0)
    return 0;
  const int nb_max = (max_seqlen_k + nsa::kBlock - 1) / nsa::kBlock;
  return nsa::selected_bwd_ws_bytes(rows_total, heads, kv_heads, k_sel, batch, nb_max);
}

nsa_status nsa_selected_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                 const void* d_out, const float* lse, nsa_dtype dtype,
                                 const int32_t* indices, int32_t k_sel,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                                 int32_t heads, int32_t kv_heads, int32_t head_dim,
                                 int32_t block_size, float softmax_scale, float* dq, float* dk,
                                 float* dv, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  const char* fn = "nsa_selected_attn_bwd";
  NSA_REQUIRE(batch >= 0 && rows_total >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(dtype == NSA_BF16, NSA_ERR_UNSUPPORTED, "%s: bfloat16 inputs only", fn);
  NSA_REQUIRE(group_ok(heads, kv_heads), NSA_ERR_UNSUPPORTED, "%s: heads %d / kv_heads %d unsupported", fn, heads, kv_heads);
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  NSA_REQUIRE(block_size == nsa::kBlock, NSA_ERR_UNSUPPORTED, "%s: block_size %d unsupported (64 only)", fn, block_size);
  NSA_REQUIRE(k_sel >= 1 && k_sel <= kMaxPrefillSel, NSA_ERR_UNSUPPORTED, "%s: k_sel %d outside 1..%d", fn, k_sel, kMaxPrefillSel);
  NSA_REQUIRE(cu_seqlens_q != nullptr, NSA_ERR_INVALID_ARG, "%s: cu_seqlens_q is required (prefill rows)", fn);
  if (rows_total == 0 || batch == 0) return ok();
  NSA_REQUIRE(max_seqlen_k >= 1, NSA_ERR_INVALID_ARG, "%s: rows without keys (max_seqlen_k 0)", fn);
  const int nb_max = (max_seqlen_k + nsa::kBlock - 1) / nsa::kBlock;
  NSA_REQUIRE(size_t(batch) * kv_heads * nb_max <= size_t(INT32_MAX) &&
                  size_t(rows_total) * kv_heads * k_sel <= size_t(INT32_MAX) &&
                  size_t(rows_total) * kv_heads <= size_t(UINT32_MAX),
              NSA_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  NSA_REQUIRE(q && k && v && out && d_out && lse && indices && cu_seqlens_k && dq && dk && dv,
              NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(d_out) &&
                  aligned16(dk) && aligned16(dv),
              NSA_ERR_INVALID_ARG, "%s: q, k, v, out, d_out, dk, dv must be 16-byte aligned", fn);
  const size_t need = nsa_selected_attn_bwd_workspace_size_min(batch, rows_total, max_seqlen_k, heads, kv_heads, k_sel);
  const size_t full = nsa_selected_attn_bwd_workspace_size(batch, rows_total, max_seqlen_k, heads, kv_heads, k_sel);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  NSA_REQUIRE(aligned16(workspace), NSA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  // dq key-block stationary when the workspace holds its partial states
  const bool blocks = workspace_bytes >= full &&
                      nsa::block_attn_grid_fits(batch, rows_total, heads, kv_heads, max_seqlen_k, k_sel);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt(float(head_dim));
  nsa::SelectedBwdArgs a{};
  a.q = static_cast<const nsa::bf16_t*>(q);
  a.k = static_cast<const nsa::bf16_t*>(k);
  a.v = static_cast<const nsa::bf16_t*>(v);
  a.out = static_cast<const nsa::bf16_t*>(out);
  a.dout = static_cast<const nsa::bf16_t*>(d_out);
  a.lse = lse;
  a.indices = indices;
  a.k_sel = k_sel;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.rows_total = rows_total;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.nb_max = nb_max;
  a.max_seqlen_k = max_seqlen_k;
  a.scale = scale;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.mode = nsa::kBwdSelected;
  a.cu_kv = cu_seqlens_k;
  nsa::selected_bwd_ws_carve(workspace, a);
  a.dq_part = blocks ? reinterpret_cast<nsa::bf16_t*>(static_cast<char*>(workspace) + ((need + 255) & ~size_t(255)))
                     : nullptr;
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_seqlens_q, batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(cu_seqlens_q, cu_seqlens_k, batch);
    chk.unique_ids(indices, long(rows_total) * kv_heads, k_sel);
  });
  return hip_status(nsa::launch_selected_bwd(a, stream), fn);
}

// ------------------------------------------- backward of the compressed and window branches

namespace {

size_t branch_bwd_ws(int32_t rows_total, int32_t heads) {
  if (rows_total <= 0 || heads <= 0) return 0;
  return (size_t(rows_total) * heads * sizeof(float) + 255) & ~size_t(255);
}

// Shared checks and launch of the two list-free branch gradients.
nsa_status branch_bwd(const char* fn, int mode, const void* q, const void* k, const void* v,
                      const void* out, const void* d_out, const float* lse, nsa_dtype dtype,
                      const int32_t* cu_q, const int32_t* cu_k, const int32_t* cu_kv,
                      int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                      int32_t max_keys, int32_t heads, int32_t kv_heads, int32_t head_dim,
                      int32_t window, float softmax_scale, int32_t accumulate, float* dq,
                      float* dk, float* dv, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  NSA_REQUIRE(batch >= 0 && rows_total >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(dtype == NSA_BF16, NSA_ERR_UNSUPPORTED, "%s: bfloat16 inputs only", fn);
  NSA_REQUIRE(group_ok(heads, kv_heads), NSA_ERR_UNSUPPORTED, "%s: heads %d / kv_heads %d unsupported", fn, heads, kv_heads);
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  NSA_REQUIRE(accumulate >= 0 && accumulate <= 3, NSA_ERR_INVALID_ARG, "%s: accumulate must be 0..3", fn);
  NSA_REQUIRE(cu_q != nullptr, NSA_ERR_INVALID_ARG, "%s: cu_seqlens_q is required (prefill rows)", fn);
  if (rows_total == 0 || batch == 0) return ok();
  NSA_REQUIRE(max_seqlen_k >= 1, NSA_ERR_INVALID_ARG, "%s: rows without keys (max_seqlen_k 0)", fn);
  const int nb_max = std::max(1, (max_keys + nsa::kBlock - 1) / nsa::kBlock);
  NSA_REQUIRE(size_t(batch) * kv_heads * nb_max <= size_t(INT32_MAX) &&
                  size_t(rows_total) * kv_heads <= size_t(UINT32_MAX),
              NSA_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  NSA_REQUIRE(q && k && v && out && d_out && lse && cu_k && cu_kv && dq && dk && dv,
              NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(d_out) &&
                  aligned16(dk) && aligned16(dv),
              NSA_ERR_INVALID_ARG, "%s: q, k, v, out, d_out, dk, dv must be 16-byte aligned", fn);
  const size_t need = branch_bwd_ws(rows_total, heads);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  nsa::SelectedBwdArgs a{};
  a.mode = mode;
  a.window = window;
  a.accumulate = accumulate;
  a.cu_kv = cu_kv;
  a.q = static_cast<const nsa::bf16_t*>(q);
  a.k = static_cast<const nsa::bf16_t*>(k);
  a.v = static_cast<const nsa::bf16_t*>(v);
  a.out = static_cast<const nsa::bf16_t*>(out);
  a.dout = static_cast<const nsa::bf16_t*>(d_out);
  a.lse = lse;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.batch = batch;
  a.rows_total = rows_total;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.nb_max = nb_max;
  a.max_seqlen_k = max_seqlen_k;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt(float(head_dim));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_q, batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(cu_q, cu_k, batch);
    if (cu_kv != cu_k) {
      chk.cu(cu_kv, batch, max_keys, nsa::kCheckCuC);
      chk.windows(cu_k, cu_kv, batch, nsa::kKernel, nsa::kStride);
    }
  });
  return hip_status(nsa::launch_selected_bwd(a, stream), fn);
}

}  // namespace

size_t nsa_branch_attn_bwd_workspace_size(int32_t rows_total, int32_t heads) {
  return branch_bwd_ws(rows_total, heads);
}

nsa_status nsa_compressed_attn_bwd(const void* q, const void* k_c, const void* v_c,
                                   const void* o_cmp, const void* d_out, const float* lse,
                                   nsa_dtype dtype, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_c,
                                   int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                                   int32_t heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t kernel, int32_t stride, float softmax_scale,
                                   int32_t accumulate, float* dq, float* dk_c, float* dv_c,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_compressed_attn_bwd";
  nsa_status st = check_geometry(fn, head_dim, kernel, stride, nsa::kBlock);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(cu_seqlens_c != nullptr || rows_total == 0 || batch == 0, NSA_ERR_INVALID_ARG,
              "%s: cu_seqlens_c is null", fn);
  return branch_bwd(fn, nsa::kBwdCompressed, q, k_c, v_c, o_cmp, d_out, lse, dtype, cu_seqlens_q,
                    cu_seqlens_k, cu_seqlens_c, batch, rows_total, max_seqlen_k,
                    nsa_window_count(max_seqlen_k, kernel, stride, 0), heads, kv_heads, head_dim,
                    0, softmax_scale, accumulate, dq, dk_c, dv_c, workspace, workspace_bytes,
                    stream);
}

nsa_status nsa_window_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                               const void* d_out, const float* lse, nsa_dtype dtype,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                               int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t window,
                               float softmax_scale, int32_t accumulate, float* dq, float* dk,
                               float* dv, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const char* fn = "nsa_window_attn_bwd";
  NSA_REQUIRE(window >= 1, NSA_ERR_INVALID_ARG, "%s: window must be >= 1", fn);
  return branch_bwd(fn, nsa::kBwdWindow, q, k, v, out, d_out, lse, dtype, cu_seqlens_q,
                    cu_seqlens_k, cu_seqlens_k, batch, rows_total, max_seqlen_k, max_seqlen_k,
                    heads, kv_heads, head_dim, window, softmax_scale, accumulate, dq, dk, dv,
                    workspace, workspace_bytes, stream);
}

nsa_status nsa_gates_bwd(const void* d_out, const void* o_cmp, const void* o_sel,
                         const void* o_win, nsa_dtype dtype, const float* gates, int32_t rows_total,
                         int32_t heads, int32_t head_dim, void* do_cmp, void* do_sel,
                         void* do_win, float* d_gates, hipStream_t stream) {
  const char* fn = "nsa_gates_bwd";
  NSA_REQUIRE(rows_total >= 0 && heads > 0, NSA_ERR_INVALID_ARG, "%s: bad rows_total or heads", fn);
  NSA_REQUIRE(dtype == NSA_BF16, NSA_ERR_UNSUPPORTED, "%s: bfloat16 only", fn);
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  if (rows_total == 0) return ok();
  NSA_REQUIRE(d_out && o_cmp && o_sel && o_win && gates && do_cmp && do_sel && do_win && d_gates,
              NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  using B = nsa::bf16_t;
  return hip_status(nsa::launch_gates_bwd(static_cast<const B*>(d_out), static_cast<const B*>(o_cmp),
                                          static_cast<const B*>(o_sel), static_cast<const B*>(o_win),
                                          gates, size_t(rows_total) * heads, static_cast<B*>(do_cmp),
                                          static_cast<B*>(do_sel), static_cast<B*>(do_win), d_gates,
                                          stream),
                    fn);
}

nsa_status nsa_compress_bwd(const float* dx_c, float* dx, const int32_t* cu_seqlens,
                            const int32_t* cu_seqlens_c, int32_t batch, int32_t max_seqlen,
                            int32_t heads, int32_t head_dim, int32_t kernel, int32_t stride,
                            int32_t accumulate, hipStream_t stream) {
  const char* fn = "nsa_compress_bwd";
  NSA_REQUIRE(batch >= 0 && max_seqlen >= 0, NSA_ERR_INVALID_ARG, "%s: negative batch or max_seqlen", fn);
  NSA_REQUIRE(heads > 0 && head_dim > 0, NSA_ERR_INVALID_ARG, "%s: heads and head_dim must be positive", fn);
  NSA_REQUIRE(kernel >= 1 && stride >= 1, NSA_ERR_INVALID_ARG, "%s: kernel and stride must be >= 1", fn);
  NSA_REQUIRE((long(heads) * head_dim) % 4 == 0 && long(heads) * head_dim < (1L << 30),
              NSA_ERR_UNSUPPORTED, "%s: heads * head_dim must be a multiple of 4", fn);
  NSA_REQUIRE(accumulate == 0 || accumulate == 1, NSA_ERR_INVALID_ARG, "%s: accumulate must be 0 or 1", fn);
  NSA_REQUIRE(batch <= 65535, NSA_ERR_UNSUPPORTED, "%s: batch above 65535", fn);
  if (batch == 0 || max_seqlen == 0) return ok();
  NSA_REQUIRE(dx_c && dx && cu_seqlens && cu_seqlens_c, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(dx_c) && aligned16(dx), NSA_ERR_INVALID_ARG, "%s: dx_c and dx must be 16-byte aligned", fn);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens, batch, max_seqlen, nsa::kCheckCuK);
    chk.cu(cu_seqlens_c, batch, -1, nsa::kCheckCuC);
    chk.windows(cu_seqlens, cu_seqlens_c, batch, kernel, stride);
  });
  return hip_status(nsa::launch_pool_bwd(dx_c, dx, cu_seqlens, cu_seqlens_c, batch, max_seqlen,
                                         heads * head_dim, kernel, stride, accumulate, stream),
                    fn);
}

// ------------------------------------------------------------------ decode step

namespace {

struct DecodeLayout {
  size_t scores, indices, attn, total;
};

DecodeLayout decode_layout(const nsa_decode_params* p) {
  DecodeLayout L{};
  const int G = p->heads / p->kv_heads;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  L.scores = 0;
  size_t off = up(nsa::scores_ws_bytes(p->batch, p->kv_heads, G, p->max_seqlen_k));
  L.indices = off;
  off += up(size_t(p->batch) * p->kv_heads * p->topk * sizeof(int32_t));
  L.attn = off;
  off += up(nsa::attn_ws_bytes(p->batch, p->kv_heads, G, p->topk, 1));
  L.total = off;
  return L;
}

nsa_status check_decode(const nsa_decode_params* p) {
  const char* fn = "nsa_decode_step";
  NSA_REQUIRE(p != nullptr, NSA_ERR_INVALID_ARG, "%s: params is null", fn);
  NSA_REQUIRE(p->batch >= 0 && p->batch <= 65535 && p->max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: bad batch or max_seqlen_k", fn);
  NSA_REQUIRE(dtype_ok(p->dtype) && dtype_ok(p->kc_dtype), NSA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  NSA_REQUIRE(group_ok(p->heads, p->kv_heads), NSA_ERR_UNSUPPORTED, "%s: heads %d / kv_heads %d unsupported", fn, p->heads, p->kv_heads);
  nsa_status st = check_geometry(fn, p->head_dim, p->kernel, p->stride, p->block_size);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(p->topk >= 1, NSA_ERR_INVALID_ARG, "%s: topk must be >= 1", fn);
  NSA_REQUIRE(p->topk <= kMaxDecodeSel, NSA_ERR_UNSUPPORTED, "%s: topk %d above the supported %d", fn, p->topk, kMaxDecodeSel);
  NSA_REQUIRE(p->n_init >= 0 && p->n_local >= 0 && p->n_init + p->n_local <= p->topk, NSA_ERR_INVALID_ARG,
              "%s: need 0 <= n_init, 0 <= n_local, n_init + n_local <= topk", fn);
  const int nb_max = (p->max_seqlen_k + p->block_size - 1) / p->block_size;
  NSA_REQUIRE(nb_max <= nsa::kMaxSortBlocks, NSA_ERR_UNSUPPORTED, "%s: %d blocks per sequence exceed the supported %d", fn, nb_max, nsa::kMaxSortBlocks);
  NSA_REQUIRE(std::isfinite(p->cis_weight), NSA_ERR_INVALID_ARG, "%s: cis_weight must be finite", fn);
  NSA_REQUIRE(p->n_cand >= 0, NSA_ERR_INVALID_ARG, "%s: n_cand must be >= 0", fn);
  if (p->batch == 0) return NSA_OK;
  NSA_REQUIRE(p->n_cand == 0 || p->cis_pooled != nullptr, NSA_ERR_INVALID_ARG,
              "%s: the two-stage choice (n_cand > 0) needs cis_pooled", fn);
  NSA_REQUIRE(p->q && p->k && p->v && p->k_c && p->cu_seqlens_k && p->cu_seqlens_c && p->out,
              NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(p->q) && aligned16(p->k) && aligned16(p->v) && aligned16(p->k_c) && aligned16(p->out),
              NSA_ERR_INVALID_ARG, "%s: q, k, v, k_c, out must be 16-byte aligned", fn);
  NSA_REQUIRE(!p->cis_values || p->cis != nullptr, NSA_ERR_INVALID_ARG, "%s: cis_values needs cis", fn);
  NSA_REQUIRE(!(p->append_window && p->cis_pooled && !p->cis), NSA_ERR_INVALID_ARG,
              "%s: refreshing cis_pooled needs cis", fn);
  return NSA_OK;
}

// Arguments of the compressed-key logits and selection launches of one decode step.
nsa::DecodeScoresArgs decode_scores_args(const nsa_decode_params* p, char* base,
                                         const DecodeLayout& lay, int32_t* idx) {
  const int G = p->heads / p->kv_heads;
  nsa::DecodeScoresArgs a{};
  a.q = p->q;
  a.q_bf16 = p->dtype == NSA_BF16;
  a.kc = p->k_c;
  a.kc_bf16 = p->kc_dtype == NSA_BF16;
  a.cis_pooled = p->cis_pooled;
  a.cis_weight = p->cis_weight;
  a.block_scores = p->block_scores;
  a.window_probs = nullptr;
  a.cu_k = p->cu_seqlens_k;
  a.cu_c = p->cu_seqlens_c;
  a.batch = p->batch;
  a.max_seqlen_k = p->max_seqlen_k;
  a.heads = p->heads;
  a.kv_heads = p->kv_heads;
  a.scale_log2 = scale_log2_of(p->softmax_scale, p->head_dim);
  a.ws = nsa::scores_ws_carve(base + lay.scores, p->batch, p->kv_heads, G, p->max_seqlen_k);
  a.indices = idx;
  a.topk = p->topk;
  a.n_init = p->n_init;
  a.n_local = p->n_local;
  a.n_cand = p->n_cand;
  if (p->append_window) {
    a.refresh_k = p->k;
    a.refresh_cis = p->cis_pooled ? p->cis : nullptr;
  }
  return a;
}

// Offloaded decode: the decode step's workspace, then the plan's slot ids, copy
// list and copy counts.
struct OffloadLayout {
  DecodeLayout dec;
  size_t slot_ids, copies, n_copy, total;
};

OffloadLayout offload_layout(const nsa_decode_params* p) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  OffloadLayout L{};
  L.dec = decode_layout(p);
  const size_t places = size_t(p->batch) * p->kv_heads * p->topk;
  L.slot_ids = L.dec.total;
  L.copies = L.slot_ids + up(places * sizeof(int32_t));
  L.n_copy = L.copies + up(places * 2 * sizeof(int32_t));
  L.total = L.n_copy + up(size_t(p->batch) * p->kv_heads * sizeof(int32_t));
  return L;
}

nsa_status check_offload_state(const char* fn, const nsa_offload_state* o) {
  NSA_REQUIRE(o != nullptr, NSA_ERR_INVALID_ARG, "%s: offload state is null", fn);
  NSA_REQUIRE(o->pool_slots >= 1 && o->pool_slots <= nsa::kMaxPoolSlots, NSA_ERR_UNSUPPORTED,
              "%s: pool_slots %d outside 1..%d", fn, o->pool_slots, nsa::kMaxPoolSlots);
  NSA_REQUIRE(o->nb_cap >= 1 && o->nb_cap <= nsa::kMaxSortBlocks, NSA_ERR_UNSUPPORTED,
              "%s: nb_cap %d outside 1..%d", fn, o->nb_cap, nsa::kMaxSortBlocks);
  NSA_REQUIRE(o->k_pool && o->v_pool && o->slot_of && o->block_of, NSA_ERR_INVALID_ARG,
              "%s: null pool or table pointer", fn);
  NSA_REQUIRE(aligned16(o->k_pool) && aligned16(o->v_pool), NSA_ERR_INVALID_ARG,
              "%s: pools must be 16-byte aligned", fn);
  return NSA_OK;
}

nsa_status check_decode_offload(const nsa_decode_params* p, const nsa_offload_state* o) {
  const char* fn = "nsa_decode_step_offload";
  nsa_status st = check_decode(p);
  if (st != NSA_OK) return st;
  st = check_offload_state(fn, o);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(p->dtype == NSA_BF16, NSA_ERR_UNSUPPORTED, "%s: bfloat16 K/V only", fn);
  NSA_REQUIRE(p->topk <= nsa::kMaxOffloadSel, NSA_ERR_UNSUPPORTED, "%s: topk %d above the supported %d", fn, p->topk, nsa::kMaxOffloadSel);
  NSA_REQUIRE(p->topk <= o->pool_slots, NSA_ERR_INVALID_ARG, "%s: pool_slots %d below topk %d", fn, o->pool_slots, p->topk);
  const int nb_max = (p->max_seqlen_k + p->block_size - 1) / p->block_size;
  NSA_REQUIRE(nb_max <= o->nb_cap, NSA_ERR_INVALID_ARG, "%s: %d blocks per sequence above nb_cap %d", fn, nb_max, o->nb_cap);
  return NSA_OK;
}

}  // namespace

size_t nsa_offload_pool_bytes(int32_t batch, int32_t kv_heads, int32_t pool_slots,
                              int32_t head_dim, nsa_dtype dtype) {
  if (batch < 0 || kv_heads <= 0 || pool_slots <= 0 || head_dim <= 0 || !dtype_ok(dtype)) return 0;
  return size_t(batch) * kv_heads * pool_slots * 64 * head_dim * (dtype == NSA_BF16 ? 2 : 4);
}

nsa_status nsa_offload_reset(const nsa_offload_state* o, int32_t batch, int32_t kv_heads,
                             hipStream_t stream) {
  const char* fn = "nsa_offload_reset";
  nsa_status st = check_offload_state(fn, o);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(batch >= 0 && kv_heads >= 1, NSA_ERR_INVALID_ARG, "%s: bad batch or kv_heads", fn);
  const size_t units = size_t(batch) * kv_heads;
  return hip_status(nsa::launch_offload_reset(o->slot_of, units * o->nb_cap, o->block_of,
                                              units * o->pool_slots, stream), fn);
}

size_t nsa_decode_offload_workspace_size(const nsa_decode_params* p, const nsa_offload_state* o) {
  if (check_decode_offload(p, o) != NSA_OK || p->batch == 0) return 0;
  return offload_layout(p).total;
}

nsa_status nsa_decode_step_offload(const nsa_decode_params* p, const nsa_offload_state* o,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_decode_step_offload";
  nsa_status st = check_decode_offload(p, o);
  if (st != NSA_OK) return st;
  if (p->batch == 0) return ok();
  const OffloadLayout lay = offload_layout(p);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= lay.total, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, lay.total);
  char* base = static_cast<char*>(workspace);
  const int G = p->heads / p->kv_heads;
  int32_t* idx = p->indices ? p->indices : reinterpret_cast<int32_t*>(base + lay.dec.indices);
  // logits and the stand-alone selection (the ids are needed before any K/V moves)
  nsa::DecodeScoresArgs a = decode_scores_args(p, base, lay.dec, idx);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(p->cu_seqlens_k, p->batch, p->max_seqlen_k, nsa::kCheckCuK);
    chk.cu(p->cu_seqlens_c, p->batch, -1, nsa::kCheckCuC);
    chk.windows(p->cu_seqlens_k, p->cu_seqlens_c, p->batch, p->kernel, p->stride);
  });
  hipError_t e = nsa::launch_decode_scores(a, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  nsa::OffloadArgs oa{};
  oa.indices = idx;
  oa.k_sel = p->topk;
  oa.units = p->batch * p->kv_heads;
  oa.kv_heads = p->kv_heads;
  oa.nb_cap = o->nb_cap;
  oa.pool_slots = o->pool_slots;
  oa.slot_of = o->slot_of;
  oa.block_of = o->block_of;
  oa.slot_ids = reinterpret_cast<int*>(base + lay.slot_ids);
  oa.copies = reinterpret_cast<int2*>(base + lay.copies);
  oa.n_copy = reinterpret_cast<int*>(base + lay.n_copy);
  oa.fetched = o->fetched;
  oa.k_src = static_cast<const nsa::bf16_t*>(p->k);
  oa.v_src = static_cast<const nsa::bf16_t*>(p->v);
  oa.cu_k = p->cu_seqlens_k;
  oa.kpool = static_cast<nsa::bf16_t*>(o->k_pool);
  oa.vpool = static_cast<nsa::bf16_t*>(o->v_pool);
  e = nsa::launch_offload_fetch(oa, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  const nsa::AttnWs aws = nsa::attn_ws_carve(base + lay.dec.attn, p->batch, p->kv_heads, G, p->topk, 1);
  e = nsa::launch_pool_attn(p->q, oa, p->cis_values ? p->cis : nullptr, p->out, p->heads,
                            a.scale_log2, aws, stream);
  return hip_status(e, fn);
}

size_t nsa_decode_workspace_size(const nsa_decode_params* p) {
  if (check_decode(p) != NSA_OK || p->batch == 0) return 0;
  return decode_layout(p).total;
}

nsa_status nsa_decode_step(const nsa_decode_params* p, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const char* fn = "nsa_decode_step";
  nsa_status st = check_decode(p);
  if (st != NSA_OK) return st;
  if (p->batch == 0) return ok();
  const DecodeLayout lay = decode_layout(p);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= lay.total, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, lay.total);
  char* base = static_cast<char*>(workspace);
  const int G = p->heads / p->kv_heads;
  int32_t* idx = p->indices ? p->indices : reinterpret_cast<int32_t*>(base + lay.indices);
  const float sl2 = scale_log2_of(p->softmax_scale, p->head_dim);
  nsa::DecodeScoresArgs a = decode_scores_args(p, base, lay, idx);
  const nsa::AttnWs aws = nsa::attn_ws_carve(base + lay.attn, p->batch, p->kv_heads, G, p->topk, 1);
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(p->cu_seqlens_k, p->batch, p->max_seqlen_k, nsa::kCheckCuK);
    chk.cu(p->cu_seqlens_c, p->batch, -1, nsa::kCheckCuC);
    chk.windows(p->cu_seqlens_k, p->cu_seqlens_c, p->batch, p->kernel, p->stride);
  });
  const int nb_max = (p->max_seqlen_k + p->block_size - 1) / p->block_size;
  if (p->dtype == NSA_BF16 && nb_max <= nsa::kFusedMaxBlocks && p->topk <= nsa::kFusedMaxSel) {
    // logits, then selection and attention in one launch, then the merge
    a.logits_only = 1;
    a.indices = p->indices;  // debug output only: the ids stay in LDS
    hipError_t e = nsa::launch_decode_scores(a, stream);
    if (e != hipSuccess) return hip_status(e, fn);
    e = nsa::launch_select_attn(a, p->k, p->v, p->cis_values ? p->cis : nullptr, p->out, aws,
                                stream);
    return hip_status(e, fn);
  }
  hipError_t e = nsa::launch_decode_scores(a, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  e = nsa::launch_selected_attn(p->q, p->k, p->v, p->dtype == NSA_BF16, idx, p->topk,
                                p->cis_values ? p->cis : nullptr, p->out, nullptr, nullptr,
                                p->cu_seqlens_k, p->batch, p->batch, p->heads, p->kv_heads, sl2,
                                aws, stream);
  return hip_status(e, fn);
}

// ----------------------------------------------------------------- prefill branches

size_t nsa_compressed_attn_workspace_size(int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                                          int32_t heads, int32_t kv_heads, int32_t kernel,
                                          int32_t stride) {
  if (batch <= 0 || rows_total <= 0 || heads <= 0 || kv_heads <= 0 || kernel < 1 || stride < 1) return 0;
  const int max_windows = nsa_window_count(max_seqlen_k, kernel, stride, 0);
  return ((size_t(rows_total) * heads * sizeof(float) + 255) & ~size_t(255)) +
         ((nsa::transposed_bytes(batch, kv_heads, max_windows) + 255) & ~size_t(255));
}

size_t nsa_window_attn_workspace_size(int32_t batch, int32_t max_seqlen_k, int32_t kv_heads) {
  if (batch <= 0 || kv_heads <= 0 || max_seqlen_k <= 0) return 0;
  return (nsa::transposed_bytes(batch, kv_heads, max_seqlen_k) + 255) & ~size_t(255);
}

}  // extern "C"

namespace {

nsa_status check_prefill_common(const char* fn, nsa_dtype dtype, int batch, int rows_total,
                                int max_seqlen_k, int heads, int kv_heads, int head_dim) {
  NSA_REQUIRE(batch >= 0 && rows_total >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(dtype == NSA_BF16, NSA_ERR_UNSUPPORTED, "%s: bfloat16 inputs only", fn);
  NSA_REQUIRE(group_ok(heads, kv_heads), NSA_ERR_UNSUPPORTED, "%s: heads %d / kv_heads %d unsupported", fn, heads, kv_heads);
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  return NSA_OK;
}

}  // namespace

extern "C" {

nsa_status nsa_compressed_attn_fwd(const void* q, const void* k_c, const void* v_c,
                                   nsa_dtype dtype, void* o_cmp, nsa_dtype out_dtype, float* lse,
                                   float* block_scores, int32_t n_blocks_max,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   const int32_t* cu_seqlens_c, int32_t batch, int32_t rows_total,
                                   int32_t max_seqlen_k, int32_t heads, int32_t kv_heads,
                                   int32_t head_dim, int32_t kernel, int32_t stride,
                                   int32_t block_size, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_compressed_attn_fwd";
  nsa_status st = check_prefill_common(fn, dtype, batch, rows_total, max_seqlen_k, heads, kv_heads, head_dim);
  if (st != NSA_OK) return st;
  st = check_geometry(fn, head_dim, kernel, stride, block_size);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(dtype_ok(out_dtype), NSA_ERR_UNSUPPORTED, "%s: unknown output dtype", fn);
  NSA_REQUIRE(cu_seqlens_q != nullptr, NSA_ERR_INVALID_ARG, "%s: cu_seqlens_q is required (prefill rows)", fn);
  if (block_scores != nullptr)
    NSA_REQUIRE(n_blocks_max >= (max_seqlen_k + block_size - 1) / block_size, NSA_ERR_INVALID_ARG,
                "%s: n_blocks_max %d < ceil(max_seqlen_k / block_size)", fn, n_blocks_max);
  if (rows_total == 0 || batch == 0) return ok();
  NSA_REQUIRE(q && k_c && v_c && o_cmp && cu_seqlens_k && cu_seqlens_c, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k_c) && aligned16(v_c) && aligned16(o_cmp), NSA_ERR_INVALID_ARG,
              "%s: q, k_c, v_c, o_cmp must be 16-byte aligned", fn);
  const size_t need = nsa_compressed_attn_workspace_size(batch, rows_total, max_seqlen_k, heads, kv_heads,
                                                        kernel, stride);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  nsa::CompressedPrefillArgs a{};
  a.q = static_cast<const nsa::bf16_t*>(q);
  a.kc = static_cast<const nsa::bf16_t*>(k_c);
  a.vc = static_cast<const nsa::bf16_t*>(v_c);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.cu_c = cu_seqlens_c;
  a.batch = batch;
  a.rows_total = rows_total;
  a.max_seqlen_q = max_seqlen_k;  // a sequence has no more query rows than keys
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.scale_log2 = scale_log2_of(softmax_scale, head_dim);
  a.max_windows = nsa_window_count(max_seqlen_k, kernel, stride, 0);
  a.lse2 = static_cast<float*>(workspace);
  a.vct = reinterpret_cast<nsa::bf16_t*>(static_cast<char*>(workspace) +
                                         ((size_t(rows_total) * heads * sizeof(float) + 255) & ~size_t(255)));
  a.o_cmp = o_cmp;
  a.out_f32 = out_dtype == NSA_F32;
  a.lse_nat = lse;
  a.block_scores = block_scores;
  a.nb_max = n_blocks_max;
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_seqlens_q, batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(cu_seqlens_q, cu_seqlens_k, batch);
    chk.cu(cu_seqlens_c, batch, -1, nsa::kCheckCuC);
    chk.windows(cu_seqlens_k, cu_seqlens_c, batch, kernel, stride);
  });
  return hip_status(nsa::launch_compressed_prefill(a, stream), fn);
}

size_t nsa_blockmask_attn_workspace_size(int32_t batch, int32_t max_seqlen, int32_t heads) {
  if (batch <= 0 || max_seqlen <= 0 || heads <= 0) return 0;
  return (nsa::transposed_bytes(batch, heads, max_seqlen) + 255) & ~size_t(255);
}

nsa_status nsa_blockmask_attn_fwd(const void* q, const void* k, const void* v, nsa_dtype dtype,
                                  const uint8_t* mask, int32_t causal, void* out,
                                  const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                                  int32_t heads, int32_t head_dim, float softmax_scale,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "nsa_blockmask_attn_fwd";
  NSA_REQUIRE(batch >= 0 && max_seqlen >= 0 && heads >= 1, NSA_ERR_INVALID_ARG, "%s: bad batch, max_seqlen or heads", fn);
  NSA_REQUIRE(dtype == NSA_BF16, NSA_ERR_UNSUPPORTED, "%s: bfloat16 inputs only", fn);
  NSA_REQUIRE(head_dim == nsa::kHeadDim, NSA_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (128 only)", fn, head_dim);
  NSA_REQUIRE(max_seqlen <= nsa::kBlockMaskMaxLen, NSA_ERR_UNSUPPORTED, "%s: max_seqlen %d above %d", fn, max_seqlen, nsa::kBlockMaskMaxLen);
  NSA_REQUIRE(heads <= 65535 && batch <= 65535, NSA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (batch == 0 || max_seqlen == 0) return ok();
  NSA_REQUIRE(q && k && v && mask && out && cu_seqlens, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), NSA_ERR_INVALID_ARG,
              "%s: q, k, v, out must be 16-byte aligned", fn);
  const size_t need = nsa_blockmask_attn_workspace_size(batch, max_seqlen, heads);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  NSA_DEVICE_CHECKS(fn, stream, chk.cu(cu_seqlens, batch, max_seqlen, nsa::kCheckCuK));
  return hip_status(nsa::launch_blockmask_attn(
                        static_cast<const nsa::bf16_t*>(q), static_cast<const nsa::bf16_t*>(k),
                        static_cast<const nsa::bf16_t*>(v), mask, causal != 0,
                        static_cast<nsa::bf16_t*>(out), cu_seqlens, batch, max_seqlen, heads,
                        scale_log2_of(softmax_scale, head_dim), static_cast<nsa::bf16_t*>(workspace),
                        stream),
                    fn);
}

nsa_status nsa_window_attn_fwd(const void* q, const void* k, const void* v, nsa_dtype dtype,
                               void* out, nsa_dtype out_dtype, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t rows_total, int32_t max_seqlen_k,
                               int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t window,
                               float softmax_scale, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const char* fn = "nsa_window_attn_fwd";
  nsa_status st = check_prefill_common(fn, dtype, batch, rows_total, max_seqlen_k, heads, kv_heads, head_dim);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(dtype_ok(out_dtype), NSA_ERR_UNSUPPORTED, "%s: unknown output dtype", fn);
  NSA_REQUIRE(window >= 1, NSA_ERR_INVALID_ARG, "%s: window must be >= 1", fn);
  NSA_REQUIRE(cu_seqlens_q != nullptr, NSA_ERR_INVALID_ARG, "%s: cu_seqlens_q is required (prefill rows)", fn);
  if (rows_total == 0 || batch == 0) return ok();
  NSA_REQUIRE(q && k && v && out && cu_seqlens_k, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), NSA_ERR_INVALID_ARG,
              "%s: q, k, v, out must be 16-byte aligned", fn);
  const size_t need = nsa_window_attn_workspace_size(batch, max_seqlen_k, kv_heads);
  NSA_REQUIRE(workspace != nullptr || need == 0, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= need, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  nsa::WindowPrefillArgs a{};
  a.q = static_cast<const nsa::bf16_t*>(q);
  a.k = static_cast<const nsa::bf16_t*>(k);
  a.v = static_cast<const nsa::bf16_t*>(v);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.rows_total = rows_total;
  a.max_seqlen_q = max_seqlen_k;
  a.max_seqlen_k = max_seqlen_k;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.window = window;
  a.vt = static_cast<nsa::bf16_t*>(workspace);
  a.scale_log2 = scale_log2_of(softmax_scale, head_dim);
  a.out = out;
  a.out_f32 = out_dtype == NSA_F32;
  a.lse_nat = lse;
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(cu_seqlens_k, batch, max_seqlen_k, nsa::kCheckCuK);
    chk.cu(cu_seqlens_q, batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(cu_seqlens_q, cu_seqlens_k, batch);
  });
  return hip_status(nsa::launch_window_prefill(a, stream), fn);
}

}  // extern "C"

namespace {

struct PrefillLayout {
  size_t lse2, vct, vt, o_cmp, o_sel, scores, indices, partial, o_sel32, base, total;
  int nb_max, max_windows;
};

PrefillLayout prefill_layout(const nsa_prefill_params* p) {
  PrefillLayout L{};
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = size_t(p->rows_total), H = size_t(p->heads);
  L.nb_max = (p->max_seqlen_k + p->block_size - 1) / p->block_size;
  L.max_windows = nsa_window_count(p->max_seqlen_k, p->kernel, p->stride, 0);
  size_t off = 0;
  L.lse2 = off;
  off += up(rows * H * sizeof(float));
  L.vct = off;
  off += up(nsa::transposed_bytes(p->batch, p->kv_heads, L.max_windows));
  L.vt = off;
  off += up(nsa::transposed_bytes(p->batch, p->kv_heads, p->max_seqlen_k));
  L.o_cmp = off;  // branch outputs kept in bf16 until the gated sum
  off += up(rows * H * p->head_dim * sizeof(uint16_t));
  L.o_sel = off;
  off += up(rows * H * p->head_dim * sizeof(uint16_t));
  L.scores = off;
  if (p->block_scores == nullptr) off += up(rows * p->kv_heads * size_t(L.nb_max) * sizeof(float));
  L.indices = off;
  if (p->indices == nullptr) off += up(rows * p->kv_heads * size_t(p->topk) * sizeof(int32_t));
  L.base = off;  // enough for the row-by-row selected branch
  // the key-block selected branch: its partial states, and its merged rows kept
  // in float32 until the gated sum (one bf16 rounding fewer, for the one its
  // partial states add)
  L.partial = off;
  off += nsa::block_attn_ws_bytes(p->rows_total, p->heads, p->kv_heads, p->topk);
  L.o_sel32 = off;
  off += up(rows * H * p->head_dim * sizeof(float));
  L.total = off;
  return L;
}

nsa_status check_prefill(const nsa_prefill_params* p) {
  const char* fn = "nsa_prefill_step";
  NSA_REQUIRE(p != nullptr, NSA_ERR_INVALID_ARG, "%s: params is null", fn);
  nsa_status st = check_prefill_common(fn, p->dtype, p->batch, p->rows_total, p->max_seqlen_k,
                                       p->heads, p->kv_heads, p->head_dim);
  if (st != NSA_OK) return st;
  st = check_geometry(fn, p->head_dim, p->kernel, p->stride, p->block_size);
  if (st != NSA_OK) return st;
  NSA_REQUIRE(p->topk >= 1 && p->topk <= kMaxPrefillSel, NSA_ERR_UNSUPPORTED, "%s: topk must be in [1, %d]", fn, kMaxPrefillSel);
  NSA_REQUIRE(p->n_init >= 0 && p->n_local >= 0 && p->n_init + p->n_local <= p->topk, NSA_ERR_INVALID_ARG,
              "%s: need 0 <= n_init, 0 <= n_local, n_init + n_local <= topk", fn);
  NSA_REQUIRE(p->window >= 1, NSA_ERR_INVALID_ARG, "%s: window must be >= 1", fn);
  NSA_REQUIRE((p->max_seqlen_k + p->block_size - 1) / p->block_size <= nsa::kMaxSortBlocks, NSA_ERR_UNSUPPORTED,
              "%s: more than %d blocks per sequence", fn, nsa::kMaxSortBlocks);
  if (p->batch == 0 || p->rows_total == 0) return NSA_OK;
  NSA_REQUIRE(p->q && p->k && p->v && p->k_c && p->v_c && p->gates && p->cu_seqlens_q && p->cu_seqlens_k &&
              p->cu_seqlens_c && p->out, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(aligned16(p->q) && aligned16(p->k) && aligned16(p->v) && aligned16(p->k_c) &&
              aligned16(p->v_c) && aligned16(p->out), NSA_ERR_INVALID_ARG,
              "%s: q, k, v, k_c, v_c, out must be 16-byte aligned", fn);
  return NSA_OK;
}

}  // namespace

extern "C" {

size_t nsa_prefill_workspace_size(const nsa_prefill_params* p) {
  if (check_prefill(p) != NSA_OK || p->batch == 0 || p->rows_total == 0) return 0;
  return prefill_layout(p).total;
}

size_t nsa_prefill_workspace_size_min(const nsa_prefill_params* p) {
  if (check_prefill(p) != NSA_OK || p->batch == 0 || p->rows_total == 0) return 0;
  return prefill_layout(p).base;
}

nsa_status nsa_prefill_step(const nsa_prefill_params* p, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const char* fn = "nsa_prefill_step";
  nsa_status st = check_prefill(p);
  if (st != NSA_OK) return st;
  if (p->batch == 0 || p->rows_total == 0) return ok();
  const PrefillLayout lay = prefill_layout(p);
  NSA_REQUIRE(workspace != nullptr, NSA_ERR_WORKSPACE, "%s: workspace is null", fn);
  NSA_REQUIRE(workspace_bytes >= lay.base, NSA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, lay.base);
  NSA_REQUIRE(aligned16(workspace), NSA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  // the key-block selected branch when the workspace holds its partial states
  const bool blocks = workspace_bytes >= lay.total &&
                      nsa::block_attn_grid_fits(p->batch, p->rows_total, p->heads, p->kv_heads, p->max_seqlen_k, p->topk);
  char* base = static_cast<char*>(workspace);
  nsa::bf16_t* o_cmp = reinterpret_cast<nsa::bf16_t*>(base + lay.o_cmp);
  nsa::bf16_t* o_sel = reinterpret_cast<nsa::bf16_t*>(base + lay.o_sel);
  float* bs = p->block_scores ? p->block_scores : reinterpret_cast<float*>(base + lay.scores);
  int32_t* idx = p->indices ? p->indices : reinterpret_cast<int32_t*>(base + lay.indices);
  const float sl2 = scale_log2_of(p->softmax_scale, p->head_dim);
  const int width = p->kv_heads * p->head_dim;
  NSA_DEVICE_CHECKS(fn, stream, {
    chk.cu(p->cu_seqlens_k, p->batch, p->max_seqlen_k, nsa::kCheckCuK);
    chk.cu(p->cu_seqlens_q, p->batch, -1, nsa::kCheckCuQ);
    chk.q_within_k(p->cu_seqlens_q, p->cu_seqlens_k, p->batch);
    chk.cu(p->cu_seqlens_c, p->batch, -1, nsa::kCheckCuC);
    chk.windows(p->cu_seqlens_k, p->cu_seqlens_c, p->batch, p->kernel, p->stride);
  });
  // 1. compressed keys and values
  hipError_t e = hipSuccess;
  if (lay.max_windows > 0) {
    e = nsa::launch_mean_pool(p->k, 1, p->k_c, 1, p->cu_seqlens_k, p->cu_seqlens_c, p->batch,
                              lay.max_windows, width, p->kernel, p->stride, 0, stream);
    if (e == hipSuccess)
      e = nsa::launch_mean_pool(p->v, 1, p->v_c, 1, p->cu_seqlens_k, p->cu_seqlens_c, p->batch,
                                lay.max_windows, width, p->kernel, p->stride, 0, stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  // 2. compressed branch and the block scores
  nsa::CompressedPrefillArgs c{};
  c.q = static_cast<const nsa::bf16_t*>(p->q);
  c.kc = static_cast<const nsa::bf16_t*>(p->k_c);
  c.vc = static_cast<const nsa::bf16_t*>(p->v_c);
  c.cu_q = p->cu_seqlens_q;
  c.cu_k = p->cu_seqlens_k;
  c.cu_c = p->cu_seqlens_c;
  c.batch = p->batch;
  c.rows_total = p->rows_total;
  c.max_seqlen_q = p->max_seqlen_k;
  c.heads = p->heads;
  c.kv_heads = p->kv_heads;
  c.scale_log2 = sl2;
  c.max_windows = lay.max_windows;
  c.lse2 = reinterpret_cast<float*>(base + lay.lse2);
  c.vct = reinterpret_cast<nsa::bf16_t*>(base + lay.vct);
  c.o_cmp = o_cmp;
  c.out_f32 = 0;
  c.lse_nat = nullptr;
  c.block_scores = bs;
  c.nb_max = lay.nb_max;
  e = nsa::launch_compressed_prefill(c, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  // 3. selection
  e = nsa::launch_select_topk(bs, idx, p->cu_seqlens_q, p->cu_seqlens_k, p->batch, p->rows_total,
                              p->kv_heads, lay.nb_max, p->topk, p->n_init, p->n_local, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  // 4. selected branch (bf16 rows)
  float* o_sel32 = blocks ? reinterpret_cast<float*>(base + lay.o_sel32) : nullptr;
  if (blocks)
    e = nsa::launch_block_attn(p->q, p->k, p->v, idx, p->topk, nullptr, nullptr, o_sel32, nullptr,
                               p->cu_seqlens_q, p->cu_seqlens_k, p->batch, p->rows_total,
                               p->heads, p->kv_heads, p->max_seqlen_k, sl2, base + lay.partial,
                               stream);
  else
    e = nsa::launch_selected_attn(p->q, p->k, p->v, 1, idx, p->topk, nullptr, o_sel, nullptr,
                                  p->cu_seqlens_q, p->cu_seqlens_k, p->batch, p->rows_total,
                                  p->heads, p->kv_heads, sl2, nsa::AttnWs{nullptr, nullptr}, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  // 5. window branch and the gated sum
  nsa::WindowPrefillArgs w{};
  w.q = c.q;
  w.k = static_cast<const nsa::bf16_t*>(p->k);
  w.v = static_cast<const nsa::bf16_t*>(p->v);
  w.cu_q = p->cu_seqlens_q;
  w.cu_k = p->cu_seqlens_k;
  w.batch = p->batch;
  w.rows_total = p->rows_total;
  w.max_seqlen_q = p->max_seqlen_k;
  w.max_seqlen_k = p->max_seqlen_k;
  w.vt = reinterpret_cast<nsa::bf16_t*>(base + lay.vt);
  w.heads = p->heads;
  w.kv_heads = p->kv_heads;
  w.window = p->window;
  w.scale_log2 = sl2;
  w.out = p->out;
  w.out_f32 = 0;
  w.lse_nat = nullptr;
  w.gates = p->gates;
  w.o_cmp = o_cmp;
  w.o_sel = o_sel;
  w.o_sel32 = o_sel32;
  return hip_status(nsa::launch_window_prefill(w, stream), fn);
}

}  // extern "C"
