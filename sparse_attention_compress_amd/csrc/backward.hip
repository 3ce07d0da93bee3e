// Backward of the selected attention (plain softmax, no CIS), prefill rows.
//
// What is computed: the gradient of the selected attention with respect to q,
// k and v for an upstream gradient dO of its output (the method is trained end
// to end: DeepSeek NSA with Triton, introduction and section 2.3, where the
// kernels are wrapped as a trainable module; the pages print no backward, so
// this is the plain gradient).  Per (row, query head h of KV group g), over the
// row's selected keys J, with p = softmax(scale K_J q) from the forward's
// log-normaliser:
//   dV_J += p dO^T,  ds = p * (V_J dO - delta),  delta = dO . O,
//   dq = scale ds K_J,  dK_J += scale ds q^T.
// dq is a gather (each row reads its own blocks).  dK and dV are sums over the
// rows that list a block; instead of scattering every (row, key) term with
// atomics, the row lists are transposed into one list of rows per (sequence,
// KV head, block) (count, scan, fill), and each block gathers its rows, in
// chunks of up to 256 rows per workgroup (the chunks of one block add their
// sums with fp32 atomics, one per gradient element and chunk).
//
// Launches: prep (delta, list counts cleared), count, scan, fill, zero (the
// blocks with long row lists), dq, dk/dv.
//
// The same kernels give the gradients of the other two prefill branches
// (DeepSeek NSA with Triton, section 1.1), whose key sets need no lists: the
// sliding-window branch (keys t - window + 1 .. t) and the compressed branch
// (the compressed windows c with 16c + 31 <= t, read from K_c and V_c).  There
// a key block is seen by one contiguous range of query positions, so the dk/dv
// workgroups walk that range directly.  `accumulate` bit 0 adds dq, bit 1 the
// key and value gradients, to what the output arrays hold, so the branches of
// one step can share dq, dk and dv.
// The order within a block's row list, and of the chunk sums, depends on
// atomics, so dK and dV are summed in an order that can change from call to
// call (fp32 rounding only).
#include <algorithm>

#include "bwd_keys.h"
#include "common.h"
#include "launch.h"

namespace nsa {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kRowsPerChunk = 256;  // rows of a block's list one dk/dv workgroup takes


// delta[row, h] = dO . O (one wave per (row, head), two dims a lane); the
// per-block row counts are cleared by the same launch.
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(
    const bf16_t* __restrict__ out, const bf16_t* __restrict__ dout, size_t n_rh,
    float* __restrict__ delta, int* __restrict__ cnt, int n_slots) {
  const int lane = threadIdx.x & 63;
  const size_t rh = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  for (size_t i = size_t(blockIdx.x) * kBwdThreads + threadIdx.x; i < size_t(n_slots);
       i += size_t(gridDim.x) * kBwdThreads)
    cnt[i] = 0;
  if (rh >= n_rh) return;
  const uint32_t o = *reinterpret_cast<const uint32_t*>(out + rh * kHeadDim + 2 * lane);
  const uint32_t d = *reinterpret_cast<const uint32_t*>(dout + rh * kHeadDim + 2 * lane);
  float s = bf16lo(o) * bf16lo(d) + bf16hi(o) * bf16hi(d);
  s = wave_reduce(s, OpSum());
  if (lane == 0) delta[rh] = s;
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

// Thread (tg, dp) of a 64-token block: tokens 4*tg .. 4*tg+3, dims 8*dp .. +7,
// kept as bf16 (one 16-byte run per token).  The 16 lanes of a DPP row hold the
// 16 dim slices of the same four tokens, so a dot product over the 128 dims is
// a row reduction, and each q or dO value read from LDS serves four keys.
struct KeyTile {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ float bf16_at(const uint4& w, int e) {
  const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return (e & 1) ? bf16hi(x) : bf16lo(x);
}

// K and V of tokens tok0 .. tok0+3 (row offsets given by the caller); a token
// with ok[i] false reads nothing and holds zeros.
__device__ __forceinline__ void load_tile(const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, const size_t off[4],
                                          const bool ok[4], KeyTile& s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s.k[i] = ok[i] ? ld16(k + off[i]) : make_uint4(0u, 0u, 0u, 0u);
    s.v[i] = ok[i] ? ld16(v + off[i]) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// The G heads' q and dO rows of one query row in LDS (fp32), with the
// log2-domain normaliser and delta.
template <int G>
struct alignas(16) RowLds {
  float q[G][kHeadDim];
  float d[G][kHeadDim];
  float lse2[G];
  float delta[G];
};

template <int G>
__device__ __forceinline__ void stage_row(RowLds<G>& R, const bf16_t* __restrict__ q,
                                          const bf16_t* __restrict__ dout,
                                          const float* __restrict__ lse,
                                          const float* __restrict__ delta, size_t head0) {
  for (int c = threadIdx.x; c < G * 16; c += kBwdThreads) {
    const int h = c >> 4, d0 = (c & 15) * 8;
    load8f(q + (head0 + h) * kHeadDim + d0, &R.q[h][d0]);
    load8f(dout + (head0 + h) * kHeadDim + d0, &R.d[h][d0]);
  }
  if (threadIdx.x < G) {
    R.lse2[threadIdx.x] = lse[head0 + threadIdx.x] * kLog2e;
    R.delta[threadIdx.x] = delta[head0 + threadIdx.x];
  }
}

// This thread's 8 dims of head h's q and dO.
template <int G>
__device__ __forceinline__ void head_slice(const RowLds<G>& R, int h, int dp, float q8[8],
                                           float d8[8]) {
  const float4 qa = *reinterpret_cast<const float4*>(&R.q[h][8 * dp]);
  const float4 qb = *reinterpret_cast<const float4*>(&R.q[h][8 * dp + 4]);
  const float4 da = *reinterpret_cast<const float4*>(&R.d[h][8 * dp]);
  const float4 db = *reinterpret_cast<const float4*>(&R.d[h][8 * dp + 4]);
  q8[0] = qa.x; q8[1] = qa.y; q8[2] = qa.z; q8[3] = qa.w;
  q8[4] = qb.x; q8[5] = qb.y; q8[6] = qb.z; q8[7] = qb.w;
  d8[0] = da.x; d8[1] = da.y; d8[2] = da.z; d8[3] = da.w;
  d8[4] = db.x; d8[5] = db.y; d8[6] = db.z; d8[7] = db.w;
}

// p and ds of head h for the thread's four tokens (every lane of the DPP row
// gets the sums over the 128 dims).
template <int G>
__device__ __forceinline__ void probs4(const RowLds<G>& R, const KeyTile& s, int h,
                                       const float q8[8], const float d8[8], const bool valid[4],
                                       float scale_log2, float p[4], float ds[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a = fmaf(q8[e], bf16_at(s.k[i], e), a);
      b = fmaf(d8[e], bf16_at(s.v[i], e), b);
    }
    a = row_reduce(a, OpSum());
    b = row_reduce(b, OpSum());
    p[i] = valid[i] ? fast_exp2(a * scale_log2 - R.lse2[h]) : 0.f;
    ds[i] = p[i] * (b - R.delta[h]);
  }
}

// dq of one (row, kv head): the row's selected blocks one at a time.  Each
// thread adds ds * k of its four tokens to its 8 dims of every head's dq in
// registers; the 16 token groups are summed once at the end (the four groups
// of a wave by lane swaps across its DPP rows, the four waves through LDS).
template <int G, int MODE>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ indices, int k_sel,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, const int* __restrict__ cu_kv,
    int window, int accumulate, int batch, int heads, int kv_heads, float scale_log2, float scale,
    float* __restrict__ dq) {
  constexpr int kOut = (G * kHeadDim + kBwdThreads - 1) / kBwdThreads;
  __shared__ RowLds<G> R;
  __shared__ float red_s[4][G][kHeadDim];
  const int tid = threadIdx.x, tg = tid >> 4, dp = tid & 15, wave = tid >> 6;
  const int row = int(blockIdx.x / unsigned(kv_heads)), g = int(blockIdx.x % unsigned(kv_heads));
  int b, t;
  bwd_row_position(row, cu_q, cu_k, batch, b, t);
  const int len = cu_k[b + 1] - cu_k[b];
  const int kstart = cu_kv[b], klen = cu_kv[b + 1] - kstart;
  const size_t head0 = size_t(row) * heads + size_t(g) * G;
  stage_row<G>(R, q, dout, lse, delta, head0);
  __syncthreads();
  const int* irow = indices + (size_t(row) * kv_heads + g) * k_sel;
  // key blocks to visit: the row's list, or the range an implicit key set covers
  int n_pl = 0, blo = 0;
  if (t >= 0 && t < len) {
    if constexpr (MODE == kBwdSelected) {
      n_pl = k_sel;
    } else if constexpr (MODE == kBwdWindow) {
      blo = max(0, t - window + 1) / kBlock;
      n_pl = t / kBlock - blo + 1;
    } else {
      const int nvis = t >= kKernel - 1 ? min(klen, (t - (kKernel - 1)) / kStride + 1) : 0;
      n_pl = (nvis + kBlock - 1) / kBlock;
    }
  }
  // at most 8 heads' accumulators at a time: a 16-head group takes two passes
  // over the blocks (the second mostly from L2) instead of one wave per SIMD
  constexpr int HG = G > 8 ? 8 : G;
#pragma unroll
  for (int h0 = 0; h0 < G; h0 += HG) {
    float acc[HG][8];
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    for (int pl = 0; pl < n_pl; ++pl) {
      int id = blo + pl;
      if constexpr (MODE == kBwdSelected) {
        id = irow[pl];
        if (id < 0 || id > t / kBlock) continue;  // uniform
      }
      bool valid[4];
      size_t off[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = kBlock * id + 4 * tg + i;
        valid[i] = key_visible<MODE>(tok, t, klen, window);
        off[i] = (size_t(kstart + min(tok, klen - 1)) * kv_heads + g) * kHeadDim + 8 * dp;
      }
      KeyTile s;
      load_tile(k, v, off, valid, s);
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        float q8[8], d8[8], p[4], ds[4];
        head_slice<G>(R, h0 + h, dp, q8, d8);
        probs4<G>(R, s, h0 + h, q8, d8, valid, scale_log2, p, ds);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ds[i], bf16_at(s.k[i], e), acc[h][e]);
      }
    }
    // sum over the token groups: the 4 DPP rows of the wave, then the 4 waves
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = cross16(acc[h][e], OpSum());
        acc[h][e] = cross32(x, OpSum());
      }
    if ((tid & 63) < 16) {
#pragma unroll
      for (int h = 0; h < HG; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) red_s[wave][h0 + h][8 * dp + e] = acc[h][e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int o = tid + kBwdThreads * i;
    if (o < G * kHeadDim) {
      const int h = o / kHeadDim, d = o % kHeadDim;
      const float x = scale * (red_s[0][h][d] + red_s[1][h][d] + red_s[2][h][d] + red_s[3][h][d]);
      if (accumulate & 1) dq[head0 * kHeadDim + o] += x; else dq[head0 * kHeadDim + o] = x;
    }
  }
}

// dK and dV of one (sequence, kv head, block) over one chunk of up to
// kRowsPerChunk of the rows that list it (grid: slot x chunk).  A block listed
// by at most one chunk's rows stores its gradients (zeros when no row lists
// it); the chunks of a longer list add theirs to the zeroed gradients with
// fp32 atomics, so the earliest blocks, which most rows list, are spread over
// several workgroups instead of one.
template <int G, int MODE>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ cnt, const int* __restrict__ off,
    const int2* __restrict__ list, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    const int* __restrict__ cu_kv, int window, int accumulate, int heads, int kv_heads,
    int nb_max, float scale_log2, float scale, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ RowLds<G> R[2];
  const int tid = threadIdx.x, tg = tid >> 4, dp = tid & 15;
  const int slot = blockIdx.x, chunk = blockIdx.y;
  const int id = slot % nb_max;
  const int g = (slot / nb_max) % kv_heads;
  const int b = slot / (nb_max * kv_heads);
  const int kstart = cu_kv[b], len = cu_kv[b + 1] - kstart;
  if (kBlock * id >= len) return;  // uniform: no key of this sequence here
  // the rows that see this block: a list (selected branch) or one range
  int n, t_lo = 0, row_lo = 0;
  if constexpr (MODE == kBwdSelected) n = cnt[slot];
  else n = implicit_rows<MODE>(b, id, len, window, cu_q, cu_k, t_lo, row_lo);
  const int e_begin = chunk * kRowsPerChunk;
  if (chunk > 0 && e_begin >= n) return;  // uniform: no rows left for this chunk
  if (n == 0 && (accumulate & 2)) return;  // nothing to add
  const int e_end = min(n, e_begin + kRowsPerChunk);
  int tok[4];
  bool tok_ok[4];
  size_t kv_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tok[i] = kBlock * id + 4 * tg + i;
    tok_ok[i] = tok[i] < len;
    kv_off[i] = (size_t(kstart + min(tok[i], len - 1)) * kv_heads + g) * kHeadDim + 8 * dp;
  }
  KeyTile s;
  load_tile(k, v, kv_off, tok_ok, s);
  float ak[4][8], av[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak[i][e] = 0.f;
      av[i][e] = 0.f;
    }
  const int first = MODE == kBwdSelected ? off[slot] : 0;
  auto entry = [&](int e) {
    if constexpr (MODE == kBwdSelected) return list[first + e];
    else return make_int2(row_lo + e, t_lo + e);
  };
  // Two listed rows (with their positions) per pair of barriers; the next
  // pair's q and dO chunks, normalisers and deltas are loaded into registers
  // while the current pair is computed.  Chunk c of a pair: row c / (16 G),
  // head (c % (16 G)) / 16, dims 8 (c % 16) .. +7.
  constexpr int kPer = (2 * G * 16 + kBwdThreads - 1) / kBwdThreads;
  uint4 pq[kPer], pd[kPer];
  float plse = 0.f, pdel = 0.f;
  int2 n0 = make_int2(0, -1), n1 = make_int2(0, -1);
  auto prefetch = [&](int e) {
    n0 = entry(e);
    n1 = e + 1 < e_end ? entry(e + 1) : n0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + kBwdThreads * i;
      if (c < 2 * G * 16) {
        const int rr = c / (G * 16), cc = c % (G * 16);
        const size_t hrow = (size_t(rr ? n1.x : n0.x) * heads + size_t(g) * G + (cc >> 4)) * kHeadDim + 8 * (cc & 15);
        pq[i] = ld16(q + hrow);
        pd[i] = ld16(dout + hrow);
      }
    }
    if (tid < 2 * G) {
      const size_t hh = size_t(tid < G ? n0.x : n1.x) * heads + size_t(g) * G + (tid % G);
      plse = lse[hh];
      pdel = delta[hh];
    }
  };
  if (e_begin < e_end) prefetch(e_begin);
  for (int e0 = e_begin; e0 < e_end; e0 += 2) {
    const bool two = e0 + 1 < e_end;  // uniform
    const int2 r0 = n0, r1 = n1;
    __syncthreads();  // the previous rows' LDS is no longer read
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + kBwdThreads * i;
      if (c < 2 * G * 16) {
        const int rr = c / (G * 16), cc = c % (G * 16);
        float* qd = &R[rr].q[cc >> 4][8 * (cc & 15)];
        float* dd = &R[rr].d[cc >> 4][8 * (cc & 15)];
        const uint32_t qw[4] = {pq[i].x, pq[i].y, pq[i].z, pq[i].w};
        const uint32_t dw[4] = {pd[i].x, pd[i].y, pd[i].z, pd[i].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          qd[2 * w] = bf16lo(qw[w]);
          qd[2 * w + 1] = bf16hi(qw[w]);
          dd[2 * w] = bf16lo(dw[w]);
          dd[2 * w + 1] = bf16hi(dw[w]);
        }
      }
    }
    if (tid < 2 * G) {
      R[tid / G].lse2[tid % G] = plse * kLog2e;
      R[tid / G].delta[tid % G] = pdel;
    }
    __syncthreads();
    if (e0 + 2 < e_end) prefetch(e0 + 2);
    for (int rr = 0; rr < (two ? 2 : 1); ++rr) {
      // An empty register barrier on the packed key tile: its bf16 -> fp32
      // conversions then stay next to their uses instead of being hoisted out
      // of the row loop as 64 more live registers (167 instead of 189 VGPRs,
      // three waves per SIMD instead of two).  It emits no instruction.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        asm volatile("" : "+v"(s.k[i].x), "+v"(s.k[i].y), "+v"(s.k[i].z), "+v"(s.k[i].w));
        asm volatile("" : "+v"(s.v[i].x), "+v"(s.v[i].y), "+v"(s.v[i].z), "+v"(s.v[i].w));
      }
      const RowLds<G>& Rr = R[rr];
      const int t = rr ? r1.y : r0.y;
      bool valid[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) valid[i] = tok_ok[i] && key_visible<MODE>(tok[i], t, len, window);
#pragma unroll 1
      for (int h = 0; h < G; ++h) {
        float q8[8], d8[8], p[4], ds[4];
        head_slice<G>(Rr, h, dp, q8, d8);
        probs4<G>(Rr, s, h, q8, d8, valid, scale_log2, p, ds);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            av[i][e] = fmaf(p[i], d8[e], av[i][e]);
            ak[i][e] = fmaf(ds[i], q8[e], ak[i][e]);
          }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!tok_ok[i]) continue;
    if (n <= kRowsPerChunk && (accumulate & 2)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dk[kv_off[i] + e] += scale * ak[i][e];
        dv[kv_off[i] + e] += av[i][e];
      }
    } else if (n <= kRowsPerChunk) {
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        *reinterpret_cast<float4*>(dk + kv_off[i] + e) =
            make_float4(scale * ak[i][e], scale * ak[i][e + 1], scale * ak[i][e + 2], scale * ak[i][e + 3]);
        *reinterpret_cast<float4*>(dv + kv_off[i] + e) =
            make_float4(av[i][e], av[i][e + 1], av[i][e + 2], av[i][e + 3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        atomicAdd(dk + kv_off[i] + e, scale * ak[i][e]);
        atomicAdd(dv + kv_off[i] + e, av[i][e]);
      }
    }
  }
}

template <int G, int MODE>
hipError_t launch_bwd_g(const SelectedBwdArgs& a, hipStream_t s) {
  const size_t n_rh = size_t(a.rows_total) * a.heads;
  const int n_slots = a.batch * a.kv_heads * a.nb_max;
  const size_t n_place = MODE == kBwdSelected ? size_t(a.rows_total) * a.kv_heads * a.k_sel : 0;
  const unsigned prep_grid = unsigned(std::max<size_t>((n_rh + 3) / 4, 1));
  hipError_t e = launch_kernel(kKindBwdLists, bwd_prep_kernel, dim3(prep_grid), dim3(kBwdThreads), s,
                               a.out, a.dout, n_rh, a.delta, a.cnt,
                               MODE == kBwdSelected ? n_slots : 0);
  if (e != hipSuccess) return e;
  const unsigned place_grid = unsigned((n_place + kBwdThreads - 1) / kBwdThreads);
  if (MODE == kBwdSelected && place_grid > 0) {
    e = launch_kernel(kKindBwdLists, bwd_count_kernel, dim3(place_grid), dim3(kBwdThreads), s,
                      a.indices, n_place, a.k_sel, a.kv_heads, a.cu_q, a.cu_k, a.batch, a.nb_max,
                      a.cnt);
    if (e != hipSuccess) return e;
  }
  if (MODE == kBwdSelected) {
    e = launch_kernel(kKindBwdLists, bwd_scan_kernel, dim3(1), dim3(kScanThreads), s,
                      static_cast<const int*>(a.cnt), n_slots, a.off, a.cursor);
    if (e != hipSuccess) return e;
  }
  if (MODE == kBwdSelected && place_grid > 0) {
    e = launch_kernel(kKindBwdLists, bwd_fill_kernel, dim3(place_grid), dim3(kBwdThreads), s,
                      a.indices, n_place, a.k_sel, a.kv_heads, a.cu_q, a.cu_k, a.batch, a.nb_max,
                      a.cursor, a.list);
    if (e != hipSuccess) return e;
  }
  // dk/dv on the matrix cores (bwd_mfma.hip), chunks of mfma_bwd_rows_per_chunk()
  // rows; the vector-ALU kernels below remain for comparison (a.valu)
  if (!(a.accumulate & 2)) {
    e = launch_kernel(kKindBwdLists, bwd_zero_kernel<MODE>, dim3(unsigned(n_slots)),
                      dim3(kBwdThreads), s, static_cast<const int*>(a.cnt), a.cu_q, a.cu_k,
                      a.cu_kv, a.window, a.kv_heads, a.nb_max,
                      a.valu ? kRowsPerChunk : mfma_bwd_rows_per_chunk(), a.dk, a.dv);
    if (e != hipSuccess) return e;
  }
  if (!a.valu) {
    if (MODE == kBwdSelected) {  // dq from the row lists on the vector ALUs, dk/dv on MFMA
      e = launch_kernel(kKindBwdQ, bwd_dq_kernel<G, MODE>,
                        dim3(unsigned(a.rows_total) * a.kv_heads), dim3(kBwdThreads), s, a.q, a.k,
                        a.v, a.dout, a.lse, static_cast<const float*>(a.delta), a.indices, a.k_sel,
                        a.cu_q, a.cu_k, a.cu_kv, a.window, a.accumulate, a.batch, a.heads,
                        a.kv_heads, a.scale * kLog2eHost, a.scale, a.dq);
      if (e != hipSuccess) return e;
    }
    return launch_bwd_mfma(a, s);
  }
  const float scale_log2 = a.scale * kLog2eHost;
  e = launch_kernel(kKindBwdQ, bwd_dq_kernel<G, MODE>, dim3(unsigned(a.rows_total) * a.kv_heads),
                    dim3(kBwdThreads), s, a.q, a.k, a.v, a.dout, a.lse,
                    static_cast<const float*>(a.delta), a.indices, a.k_sel, a.cu_q, a.cu_k,
                    a.cu_kv, a.window, a.accumulate, a.batch, a.heads, a.kv_heads, scale_log2,
                    a.scale, a.dq);
  if (e != hipSuccess) return e;
  // the most rows one key block can have: every row (selected, compressed) or
  // the 64 + window - 1 positions that see a block of the window branch
  const int max_rows = MODE == kBwdWindow ? std::min(a.max_seqlen_k, kBlock + a.window - 1)
                                          : a.max_seqlen_k;
  const unsigned n_chunk = unsigned((max_rows + kRowsPerChunk - 1) / kRowsPerChunk);
  return launch_kernel(kKindBwdKV, bwd_dkdv_kernel<G, MODE>,
                       dim3(unsigned(n_slots), std::max(1u, n_chunk)), dim3(kBwdThreads), s, a.q,
                       a.k, a.v, a.dout, a.lse, static_cast<const float*>(a.delta),
                       static_cast<const int*>(a.cnt), static_cast<const int*>(a.off),
                       static_cast<const int2*>(a.list), a.cu_q, a.cu_k, a.cu_kv, a.window,
                       a.accumulate, a.heads, a.kv_heads, a.nb_max, scale_log2, a.scale, a.dk,
                       a.dv);
}

template <int MODE>
hipError_t launch_bwd_mode(const SelectedBwdArgs& a, hipStream_t s) {
  switch (a.heads / a.kv_heads) {
    case 1: return launch_bwd_g<1, MODE>(a, s);
    case 2: return launch_bwd_g<2, MODE>(a, s);
    case 4: return launch_bwd_g<4, MODE>(a, s);
    case 8: return launch_bwd_g<8, MODE>(a, s);
    case 16: return launch_bwd_g<16, MODE>(a, s);
    default: return hipErrorInvalidValue;
  }
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
    case kBwdSelected: return launch_bwd_mode<kBwdSelected>(a, s);
    case kBwdWindow: return launch_bwd_mode<kBwdWindow>(a, s);
    case kBwdCompressed: return launch_bwd_mode<kBwdCompressed>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Gradients of the gated sum o = g0 o_cmp + g1 o_sel + g2 o_win: each branch's
// output gradient g_b dO (bf16) and dg_b = dO . o_b (fp32); one wave per (row,
// head), two dims a lane.
__global__ __launch_bounds__(256) void gates_bwd_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ o_cmp,
    const bf16_t* __restrict__ o_sel, const bf16_t* __restrict__ o_win,
    const float* __restrict__ gates, size_t n_rh, bf16_t* __restrict__ do_cmp,
    bf16_t* __restrict__ do_sel, bf16_t* __restrict__ do_win, float* __restrict__ d_gates) {
  const int lane = threadIdx.x & 63;
  const size_t rh = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (rh >= n_rh) return;
  const size_t o = rh * kHeadDim + 2 * lane;
  const uint32_t d = *reinterpret_cast<const uint32_t*>(dout + o);
  const float d0 = bf16lo(d), d1 = bf16hi(d);
  const bf16_t* ob[3] = {o_cmp, o_sel, o_win};
  bf16_t* db[3] = {do_cmp, do_sel, do_win};
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const float g = gates[rh * 3 + j];
    const uint32_t x = *reinterpret_cast<const uint32_t*>(ob[j] + o);
    float s = d0 * bf16lo(x) + d1 * bf16hi(x);
    s = wave_reduce(s, OpSum());
    *reinterpret_cast<uint32_t*>(db[j] + o) = pack_bf16x2(g * d0, g * d1);
    if (lane == 0) d_gates[rh * 3 + j] = s;
  }
}

hipError_t launch_gates_bwd(const bf16_t* dout, const bf16_t* o_cmp, const bf16_t* o_sel,
                            const bf16_t* o_win, const float* gates, size_t n_rh, bf16_t* do_cmp,
                            bf16_t* do_sel, bf16_t* do_win, float* d_gates, hipStream_t s) {
  if (n_rh == 0) return hipSuccess;
  return launch_kernel(kKindBwdLists, gates_bwd_kernel, dim3(unsigned((n_rh + 3) / 4)), dim3(256),
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
