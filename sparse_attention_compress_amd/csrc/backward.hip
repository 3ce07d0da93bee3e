// Backward of the prefill branches: the host-side launcher and the list and
// elementwise kernels around the matrix-core gradient kernels of bwd_mfma.hip.
//
// What is computed: the gradient of a branch's attention with respect to q, k
// and v for an upstream gradient dO of its output (the method is trained end
// to end: DeepSeek NSA with Triton, introduction and section 2.3, where the
// kernels are wrapped as a trainable module; the pages print no backward, so
// this is the plain gradient).  Per (row, query head h of KV group g), over the
// row's keys J, with p = softmax(scale K_J q) from the forward's
// log-normaliser:
//   dV_J += p dO^T,  ds = p * (V_J dO - delta),  delta = dO . O,
//   dq = scale ds K_J,  dK_J += scale ds q^T.
// Key sets (section 1.1): the tokens of the row's listed blocks (selected
// branch), the last `window` tokens (sliding-window branch), the compressed
// windows visible to the row (compressed branch; k, v are then K_c, V_c).
//
// dK and dV are gathered per (sequence, KV head, 64-key block) over the rows
// that see the block.  For the selected branch the row lists are transposed
// into one list of rows per block (count, scan, fill); for the other two the
// rows that see a block form one contiguous range of positions and need no
// list.  A block seen by more rows than one workgroup takes is cleared first
// (zero) and its chunks add their sums with fp32 atomics, so dK and dV are
// summed in an order that can change from call to call (fp32 rounding only).
// `accumulate` bit 0 adds dq, bit 1 the key and value gradients, to what the
// output arrays hold, so the branches of one step can share dq, dk and dv.
//
// Launches: prep (delta, list counts cleared), count, scan, fill (selected
// branch; count and fill per chunk of rows with LDS tables, or per place for
// sequences of more than 8192 blocks), zero, then the matrix-core dk/dv and dq
// kernels.  Also here: the
// window mean's transpose (dK_c, dV_c back onto K, V) and the gradients of the
// gated sum of the three branches.
#include <algorithm>

#include "bwd_keys.h"
#include "common.h"
#include "launch.h"

namespace nsa {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kScanThreads = 1024;


// Dot product of two rows' 8-dim pieces (bf16).
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b) {
  float s = bf16lo(a.x) * bf16lo(b.x);
  s = fmaf(bf16hi(a.x), bf16hi(b.x), s);
  s = fmaf(bf16lo(a.y), bf16lo(b.y), s);
  s = fmaf(bf16hi(a.y), bf16hi(b.y), s);
  s = fmaf(bf16lo(a.z), bf16lo(b.z), s);
  s = fmaf(bf16hi(a.z), bf16hi(b.z), s);
  s = fmaf(bf16lo(a.w), bf16lo(b.w), s);
  return fmaf(bf16hi(a.w), bf16hi(b.w), s);
}

// (row, head) pairs per 256-thread workgroup of the row-dot kernels: 16 lanes
// (one DPP row) a pair, 8 dims a lane, so every load is 16 bytes.
constexpr int kRhPerWg = kBwdThreads / 16;

// delta[row, h] = dO . O; the per-block row counts are cleared by the same
// launch.
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(
    const bf16_t* __restrict__ out, const bf16_t* __restrict__ dout, size_t n_rh,
    float* __restrict__ delta, int* __restrict__ cnt, int n_slots) {
  const int sub = threadIdx.x & 15;
  const size_t rh = size_t(blockIdx.x) * kRhPerWg + (threadIdx.x >> 4);
  for (size_t i = size_t(blockIdx.x) * kBwdThreads + threadIdx.x; i < size_t(n_slots);
       i += size_t(gridDim.x) * kBwdThreads)
    cnt[i] = 0;
  if (rh >= n_rh) return;  // whole rows of 16 lanes
  const size_t o = rh * kHeadDim + 8 * sub;
  const float s = row_reduce(dot8_bf16(ld16(out + o), ld16(dout + o)), OpSum());
  if (sub == 0) delta[rh] = s;
}

// One thread per (row, kv head, place): whether the place lists a block the
// row attends to, its (sequence, kv head, block) slot, and the row's position.
__device__ __forceinline__ int bwd_slot_of(size_t i, const int* __restrict__ indices, int k_sel,
                                           int kv_heads, const int* __restrict__ cu_q,
                                           const int* __restrict__ cu_k, int batch, int nb_max,
                                           int& row, int& t) {
  const size_t unit = i / size_t(k_sel);
  row = int(unit / size_t(kv_heads));
  const int g = int(unit % size_t(kv_heads));
  const int id = indices[i];
  t = -1;
  if (id < 0 || id >= nb_max) return -1;
  int b;
  bwd_row_position(row, cu_q, cu_k, batch, b, t);
  const int len = cu_k[b + 1] - cu_k[b];
  if (t < 0 || t >= len || kBlock * id > t) return -1;
  return (b * kv_heads + g) * nb_max + id;
}

__global__ __launch_bounds__(kBwdThreads) void bwd_count_kernel(
    const int* __restrict__ indices, size_t n, int k_sel, int kv_heads,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int nb_max,
    int* __restrict__ cnt) {
  const size_t i = size_t(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (i >= n) return;
  int row, t;
  const int slot = bwd_slot_of(i, indices, k_sel, kv_heads, cu_q, cu_k, batch, nb_max, row, t);
  if (slot >= 0) atomicAdd(cnt + slot, 1);
}

// Exclusive scan of the counts into the list offsets (and the fill cursors),
// one workgroup walking the slots 1024 at a time.
__global__ __launch_bounds__(kScanThreads) void bwd_scan_kernel(const int* __restrict__ cnt,
                                                                int n_slots, int* __restrict__ off,
                                                                int* __restrict__ cursor) {
  __shared__ int wsum[kScanThreads / kWave];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n_slots; base += kScanThreads) {
    const int i = base + tid;
    const int c = i < n_slots ? cnt[i] : 0;
    const int incl = wave_inclusive_scan(c);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - c;
    if (i < n_slots) {
      off[i] = excl;
      cursor[i] = excl;
    }
    __syncthreads();
    if (tid == kScanThreads - 1) carry_s = excl + c;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBwdThreads) void bwd_fill_kernel(
    const int* __restrict__ indices, size_t n, int k_sel, int kv_heads,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int nb_max,
    int* __restrict__ cursor, int2* __restrict__ list) {
  const size_t i = size_t(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (i >= n) return;
  int row, t;
  const int slot = bwd_slot_of(i, indices, k_sel, kv_heads, cu_q, cu_k, batch, nb_max, row, t);
  if (slot >= 0) list[atomicAdd(cursor + slot, 1)] = make_int2(row, t);
}

// The same counts and lists built per (sequence, KV head, chunk of kListRows
// query rows): a chunk's places are first counted per block in LDS, so the
// global counters and cursors take one atomic per (chunk, block) instead of one
// per place (the places of a row's early blocks otherwise all hit one counter).
// Used when a sequence's blocks fit the LDS table.
constexpr int kListRows = 1024;
constexpr int kListMaxBlocks = 8192;

// The chunk's places (rows r0 .. r1 - 1 of sequence b, KV head kv) that list a
// block the row attends to: f(row, t, id) for each.
template <typename F>
__device__ __forceinline__ void for_chunk_places(const int* __restrict__ indices, int k_sel,
                                                 int kv_heads, int kv, int q0, int r0, int r1,
                                                 int off, int nb_max, F f) {
  const int n = (r1 - r0) * k_sel;
  for (int p = threadIdx.x; p < n; p += kBwdThreads) {
    const int dr = p / k_sel, r = r0 + dr, place = p - dr * k_sel;
    const int id = indices[(size_t(q0 + r) * kv_heads + kv) * k_sel + place];
    const int t = r + off;
    if (id >= 0 && id < nb_max && kBlock * id <= t) f(q0 + r, t, id);
  }
}

// FILL = false: add the chunk's per-block counts to cnt.  FILL = true: reserve
// each block's range at its cursor, then write the chunk's entries (row, t)
// into it.  Grid (chunk, KV head, sequence).
template <bool FILL>
__global__ __launch_bounds__(kBwdThreads) void bwd_chunk_lists_kernel(
    const int* __restrict__ indices, int k_sel, int kv_heads, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int nb_max, int* __restrict__ counters,
    int2* __restrict__ list) {
  __shared__ int h[kListMaxBlocks];
  const int c = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int q0 = cu_q[b], lq = cu_q[b + 1] - q0;
  const int r0 = c * kListRows;
  if (r0 >= lq) return;  // the same for the whole workgroup
  const int r1 = min(lq, r0 + kListRows);
  const int off = (cu_k[b + 1] - cu_k[b]) - lq;
  // the chunk's rows list ids up to (r1 - 1 + off) / 64
  const int nb = min(nb_max, max(0, r1 - 1 + off) / kBlock + 1);
  for (int i = threadIdx.x; i < nb; i += kBwdThreads) h[i] = 0;
  __syncthreads();
  for_chunk_places(indices, k_sel, kv_heads, kv, q0, r0, r1, off, nb_max,
                   [&](int, int, int id) { atomicAdd(&h[id], 1); });
  __syncthreads();
  int* g = counters + size_t(b * kv_heads + kv) * nb_max;
  for (int i = threadIdx.x; i < nb; i += kBwdThreads) {
    const int n = h[i];
    if constexpr (FILL) h[i] = n ? atomicAdd(g + i, n) : 0;
    else if (n) atomicAdd(g + i, n);
  }
  if constexpr (FILL) {
    __syncthreads();
    for_chunk_places(indices, k_sel, kv_heads, kv, q0, r0, r1, off, nb_max,
                     [&](int row, int t, int id) { list[atomicAdd(&h[id], 1)] = make_int2(row, t); });
  }
}

// dk and dv of the blocks whose row list spans several chunks start at 0 (the
// chunks add to them); one workgroup per (sequence, kv head, block).
template <int MODE>
__global__ __launch_bounds__(kBwdThreads) void bwd_zero_kernel(
    const int* __restrict__ cnt, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    const int* __restrict__ cu_kv, int window, int kv_heads, int nb_max, int rows_per_chunk,
    float* __restrict__ dk, float* __restrict__ dv) {
  const int slot = blockIdx.x;
  const int id = slot % nb_max;
  const int g = (slot / nb_max) % kv_heads;
  const int b = slot / (nb_max * kv_heads);
  const int kstart = cu_kv[b], len = cu_kv[b + 1] - kstart;
  if (kBlock * id >= len) return;
  int n;
  if constexpr (MODE == kBwdSelected) {
    n = cnt[slot];
  } else {
    int t_lo, row_lo;
    n = implicit_rows<MODE>(b, id, len, window, cu_q, cu_k, t_lo, row_lo);
  }
  if (n <= rows_per_chunk) return;
  const int tok = kBlock * id + (threadIdx.x >> 2);
  if (tok >= len) return;
  const size_t o = (size_t(kstart + tok) * kv_heads + g) * kHeadDim + 32 * (threadIdx.x & 3);
#pragma unroll
  for (int e = 0; e < 32; e += 4) {
    *reinterpret_cast<float4*>(dk + o + e) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dv + o + e) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int MODE>
hipError_t launch_bwd_lists(const SelectedBwdArgs& a, hipStream_t s) {
  const size_t n_rh = size_t(a.rows_total) * a.heads;
  const int n_slots = a.batch * a.kv_heads * a.nb_max;
  const size_t n_place = MODE == kBwdSelected ? size_t(a.rows_total) * a.kv_heads * a.k_sel : 0;
  const unsigned prep_grid = unsigned(std::max<size_t>((n_rh + kRhPerWg - 1) / kRhPerWg, 1));
  hipError_t e = launch_kernel(kKindBwdLists, bwd_prep_kernel, dim3(prep_grid), dim3(kBwdThreads), s,
                               a.out, a.dout, n_rh, a.delta, a.cnt,
                               MODE == kBwdSelected ? n_slots : 0);
  if (e != hipSuccess) return e;
  const unsigned place_grid = unsigned((n_place + kBwdThreads - 1) / kBwdThreads);
  // per-chunk counting (LDS first) when the blocks fit its table, else per place
  const bool chunked = a.nb_max <= kListMaxBlocks;
  const dim3 chunk_grid(unsigned((a.max_seqlen_k + kListRows - 1) / kListRows),
                        unsigned(a.kv_heads), unsigned(a.batch));
  if (MODE == kBwdSelected && place_grid > 0) {
    e = chunked ? launch_kernel(kKindBwdLists, bwd_chunk_lists_kernel<false>, chunk_grid,
                                dim3(kBwdThreads), s, a.indices, a.k_sel, a.kv_heads, a.cu_q,
                                a.cu_k, a.nb_max, a.cnt, static_cast<int2*>(nullptr))
                : launch_kernel(kKindBwdLists, bwd_count_kernel, dim3(place_grid),
                                dim3(kBwdThreads), s, a.indices, n_place, a.k_sel, a.kv_heads,
                                a.cu_q, a.cu_k, a.batch, a.nb_max, a.cnt);
    if (e != hipSuccess) return e;
  }
  if (MODE == kBwdSelected) {
    e = launch_kernel(kKindBwdLists, bwd_scan_kernel, dim3(1), dim3(kScanThreads), s,
                      static_cast<const int*>(a.cnt), n_slots, a.off, a.cursor);
    if (e != hipSuccess) return e;
  }
  if (MODE == kBwdSelected && place_grid > 0) {
    e = chunked ? launch_kernel(kKindBwdLists, bwd_chunk_lists_kernel<true>, chunk_grid,
                                dim3(kBwdThreads), s, a.indices, a.k_sel, a.kv_heads, a.cu_q,
                                a.cu_k, a.nb_max, a.cursor, a.list)
                : launch_kernel(kKindBwdLists, bwd_fill_kernel, dim3(place_grid),
                                dim3(kBwdThreads), s, a.indices, n_place, a.k_sel, a.kv_heads,
                                a.cu_q, a.cu_k, a.batch, a.nb_max, a.cursor, a.list);
    if (e != hipSuccess) return e;
  }
  // dk/dv and dq on the matrix cores (bwd_mfma.hip); blocks seen by more rows
  // than one dk/dv workgroup takes are cleared first and summed with atomics
  if (!(a.accumulate & 2)) {
    e = launch_kernel(kKindBwdLists, bwd_zero_kernel<MODE>, dim3(unsigned(n_slots)),
                      dim3(kBwdThreads), s, static_cast<const int*>(a.cnt), a.cu_q, a.cu_k,
                      a.cu_kv, a.window, a.kv_heads, a.nb_max, mfma_bwd_rows_per_chunk(MODE), a.dk,
                      a.dv);
    if (e != hipSuccess) return e;
  }
  return launch_bwd_mfma(a, s);
}

// dx[j] (+)= sum over the windows c that hold token j of dx_c[c] / (valid tokens
// of c): the transpose of the window mean.  One thread per 4 channels of one
// token row; the grid's y dimension is the sequence.
__global__ __launch_bounds__(256) void pool_bwd_kernel(const float* __restrict__ dxc,
                                                       float* __restrict__ dx,
                                                       const int* __restrict__ cu,
                                                       const int* __restrict__ cu_c, int width,
                                                       int kernel, int stride, int accumulate) {
  const int b = blockIdx.y;
  const int start = cu[b], len = cu[b + 1] - start;
  const int cstart = cu_c[b], nc = cu_c[b + 1] - cstart;
  const int w4 = width / 4;
  const long i = long(blockIdx.x) * 256 + threadIdx.x;
  if (i >= long(len) * w4) return;
  const int j = int(i / w4), ch = 4 * int(i % w4);
  // windows c with stride*c <= j < stride*c + kernel, 0 <= c < nc
  const int c_lo = j >= kernel ? (j - kernel) / stride + 1 : 0;
  const int c_hi = min(nc - 1, j / stride);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = c_lo; c <= c_hi; ++c) {
    const float inv = 1.f / float(min(kernel, len - stride * c));
    const float4 g = *reinterpret_cast<const float4*>(dxc + size_t(cstart + c) * width + ch);
    acc.x += g.x * inv;
    acc.y += g.y * inv;
    acc.z += g.z * inv;
    acc.w += g.w * inv;
  }
  float4* o = reinterpret_cast<float4*>(dx + size_t(start + j) * width + ch);
  if (accumulate) {
    const float4 x = *o;
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  *o = acc;
}

}  // namespace

size_t selected_bwd_ws_bytes(int rows_total, int heads, int kv_heads, int k_sel, int batch,
                             int nb_max) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_slots = size_t(batch) * kv_heads * nb_max;
  return up(size_t(rows_total) * heads * sizeof(float)) + 3 * up(n_slots * sizeof(int)) +
         up(size_t(rows_total) * kv_heads * k_sel * sizeof(int2));
}

void selected_bwd_ws_carve(void* base, SelectedBwdArgs& a) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_slots = size_t(a.batch) * a.kv_heads * a.nb_max;
  char* p = static_cast<char*>(base);
  a.delta = reinterpret_cast<float*>(p);
  p += up(size_t(a.rows_total) * a.heads * sizeof(float));
  a.cnt = reinterpret_cast<int*>(p);
  p += up(n_slots * sizeof(int));
  a.off = reinterpret_cast<int*>(p);
  p += up(n_slots * sizeof(int));
  a.cursor = reinterpret_cast<int*>(p);
  p += up(n_slots * sizeof(int));
  a.list = reinterpret_cast<int2*>(p);
}

hipError_t launch_selected_bwd(const SelectedBwdArgs& a, hipStream_t s) {
  switch (a.mode) {
    case kBwdSelected: return launch_bwd_lists<kBwdSelected>(a, s);
    case kBwdWindow: return launch_bwd_lists<kBwdWindow>(a, s);
    case kBwdCompressed: return launch_bwd_lists<kBwdCompressed>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Gradients of the gated sum o = g0 o_cmp + g1 o_sel + g2 o_win: each branch's
// output gradient g_b dO (bf16) and dg_b = dO . o_b (fp32); one wave per (row,
// head), two dims a lane.
__global__ __launch_bounds__(kBwdThreads) void gates_bwd_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ o_cmp,
    const bf16_t* __restrict__ o_sel, const bf16_t* __restrict__ o_win,
    const float* __restrict__ gates, size_t n_rh, bf16_t* __restrict__ do_cmp,
    bf16_t* __restrict__ do_sel, bf16_t* __restrict__ do_win, float* __restrict__ d_gates) {
  const int sub = threadIdx.x & 15;
  const size_t rh = size_t(blockIdx.x) * kRhPerWg + (threadIdx.x >> 4);
  if (rh >= n_rh) return;  // whole rows of 16 lanes
  const size_t o = rh * kHeadDim + 8 * sub;
  const uint4 d = ld16(dout + o);
  const bf16_t* ob[3] = {o_cmp, o_sel, o_win};
  bf16_t* db[3] = {do_cmp, do_sel, do_win};
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const float g = gates[rh * 3 + j];
    const float s = row_reduce(dot8_bf16(d, ld16(ob[j] + o)), OpSum());
    *reinterpret_cast<uint4*>(db[j] + o) =
        make_uint4(pack_bf16x2(g * bf16lo(d.x), g * bf16hi(d.x)), pack_bf16x2(g * bf16lo(d.y), g * bf16hi(d.y)),
                   pack_bf16x2(g * bf16lo(d.z), g * bf16hi(d.z)), pack_bf16x2(g * bf16lo(d.w), g * bf16hi(d.w)));
    if (sub == 0) d_gates[rh * 3 + j] = s;
  }
}

hipError_t launch_gates_bwd(const bf16_t* dout, const bf16_t* o_cmp, const bf16_t* o_sel,
                            const bf16_t* o_win, const float* gates, size_t n_rh, bf16_t* do_cmp,
                            bf16_t* do_sel, bf16_t* do_win, float* d_gates, hipStream_t s) {
  if (n_rh == 0) return hipSuccess;
  return launch_kernel(kKindBwdLists, gates_bwd_kernel, dim3(unsigned((n_rh + kRhPerWg - 1) / kRhPerWg)), dim3(kBwdThreads),
                       s, dout, o_cmp, o_sel, o_win, gates, n_rh, do_cmp, do_sel, do_win, d_gates);
}

hipError_t launch_pool_bwd(const float* dxc, float* dx, const int* cu, const int* cu_c, int batch,
                           int n_tokens_max, int width, int kernel, int stride, int accumulate,
                           hipStream_t s) {
  const long items = long(n_tokens_max) * (width / 4);
  const unsigned gx = unsigned((items + 255) / 256);
  if (gx == 0 || batch == 0) return hipSuccess;
  return launch_kernel(kKindPool, pool_bwd_kernel, dim3(gx, unsigned(batch)), dim3(256), s, dxc,
                       dx, cu, cu_c, width, kernel, stride, accumulate);
}

}  // namespace nsa
