// Prefill branches of native sparse attention: compressed attention (with the
// group-summed probabilities max-pooled onto blocks for the selection) and
// sliding-window attention (with the gated sum of the three branches).
//
// What is computed (DeepSeek NSA with Triton, section 1.1: three branches summed
// with per-token, per-head gates; the selection reuses the compressed-attention
// probabilities; the window covers the last 512 tokens):
//   o_cmp(t, h) = softmax over visible windows c of scale * q_h . Kc[c], times Vc
//                 (window c visible when its last token 16c+31 <= t);
//   block score(t, g, i) = max over windows c overlapping block i of
//                 sum over heads h of group g of P_h(t, c)  (windows 4i-1..4i+3);
//   o_win(t, h) = softmax over keys max(0, t-W+1) .. t, times V;
//   o(t, h)     = g0 o_cmp + g1 o_sel + g2 o_win.
//
// Design (gfx950): one wave per query token and KV group; the group's G <= 16
// query heads are the 16 columns of the MFMA tiles, keys (or windows) go 16 at a
// time as the rows: S^T = K Q^T with four v_mfma_f32_16x16x32_bf16 (key rows
// loaded straight into the A operand, Q^T kept in registers), then
// O^T += V^T P^T with eight v_mfma_f32_16x16x16_bf16 (P^T is already in the
// operand layout).  A workgroup holds 4 waves = 4 consecutive tokens of one KV
// group, so the key tiles they share are served from L1/L2.  No LDS, no
// workgroup barriers.  The compressed branch runs in two passes: the first finds
// each head's log2 normaliser, the second forms normalised probabilities, which
// give o_cmp directly and, summed over the 16 head columns with DPP, the window
// scores of the group.
#include "common.h"
#include "launch.h"

namespace nsa {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void prefill_row_position(int row, const int* __restrict__ cu_q,
                                                     const int* __restrict__ cu_k, int batch,
                                                     int& b, int& t) {
  int lo = 0, hi = batch - 1;  // last sequence whose first row is <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  b = lo;
  t = (row - cu_q[b]) + ((cu_k[b + 1] - cu_k[b]) - (cu_q[b + 1] - cu_q[b]));
}

__device__ __forceinline__ uint32_t ld_h(const bf16_t* p) {
  return uint32_t(*reinterpret_cast<const uint16_t*>(p));
}

// One 16-key tile of a wave: keys key0 + r (r < 16) of rows `base + key*rs`.
// ka: A operand of S^T = K Q^T (key c16, dims 32i + 8 r4 .. +8).
// va: A operand of O^T = V^T P^T (dim 16n + c16; keys 4 r4 + 2m, +1).
// Key rows are clamped to [0, kmax] so every load is in bounds; the caller masks.
struct KeyTile {
  uint4 ka[4];
  uint32_t va[16];
};

template <bool WITH_V>
__device__ __forceinline__ void load_tile(const bf16_t* __restrict__ kb, const bf16_t* __restrict__ vb,
                                          size_t rs, int key0, int kmax, KeyTile& T) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
  const bf16_t* kr = kb + size_t(min(key0 + c16, kmax)) * rs + 8 * r4;
#pragma unroll
  for (int i = 0; i < 4; ++i) T.ka[i] = ld16(kr + 32 * i);
  if constexpr (WITH_V) {
    const bf16_t* vr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vr[e] = vb + size_t(min(key0 + 4 * r4 + e, kmax)) * rs + c16;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        T.va[2 * n + m] = ld_h(vr[2 * m] + 16 * n) | (ld_h(vr[2 * m + 1] + 16 * n) << 16);
  }
}

__device__ __forceinline__ f32x4_t tile_scores(const KeyTile& T, const uint4 (&qb)[4]) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, T.ka[i]),
                                                __builtin_bit_cast(bf16x8_t, qb[i]), s, 0, 0, 0);
  return s;
}

__device__ __forceinline__ void tile_pv(const KeyTile& T, const float (&p)[4], f32x4_t (&acc)[8]) {
  const bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
  const bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
  const s16x4_t pb = __builtin_bit_cast(
      s16x4_t, make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)));
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const s16x4_t va = __builtin_bit_cast(s16x4_t, make_uint2(T.va[2 * n], T.va[2 * n + 1]));
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[n], 0, 0, 0);
  }
}

// Column (head) reductions over the 4 lane rows of a wave.
__device__ __forceinline__ float rows_max(float x) { return cross32(cross16(x, OpMax()), OpMax()); }
__device__ __forceinline__ float rows_sum(float x) { return cross32(cross16(x, OpSum()), OpSum()); }

// B operand of S^T = K Q^T for query row `qrow` (heads of one group): Q^T[dims
// 32i + 8 r4 .. +8][head c16], zero past G.
template <int G>
__device__ __forceinline__ void load_q(const bf16_t* __restrict__ qrow, uint4 (&qb)[4]) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
  const bf16_t* qp = qrow + size_t(min(c16, G - 1)) * kHeadDim + 8 * r4;
#pragma unroll
  for (int i = 0; i < 4; ++i) qb[i] = ld16(qp + 32 * i);
  if (c16 >= G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Store the lane's O^T entries (head c16, dims 16n + 4 r4 .. +3) scaled by `f`.
template <int G>
__device__ __forceinline__ void store_rows(void* __restrict__ out, int out_f32, size_t head0,
                                           const f32x4_t (&acc)[8], float f) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
  if (c16 >= G) return;
  const size_t o = (head0 + c16) * kHeadDim + 4 * r4;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    if (out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + o + 16 * n) =
          make_float4(acc[n][0] * f, acc[n][1] * f, acc[n][2] * f, acc[n][3] * f);
    } else {
      bf16_t* dst = static_cast<bf16_t*>(out) + o + 16 * n;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[n][0] * f, acc[n][1] * f),
                                                  pack_bf16x2(acc[n][2] * f, acc[n][3] * f));
    }
  }
}

// ------------------------------------------------------------- compressed branch

// PROBS = false: per (row, head) log2 normaliser lse2 = max + log2(sum exp2).
// PROBS = true:  o_cmp, natural-log lse, and the group's block scores.
template <int G, bool PROBS>
__global__ __launch_bounds__(256) void compressed_prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, const int* __restrict__ cu_c,
    int batch, int rows_total, int kv_heads, float scale_log2, float* __restrict__ lse2,
    void* __restrict__ o_cmp, int out_f32, float* __restrict__ lse_nat,
    float* __restrict__ block_scores, int nb_max) {
  constexpr int D = kHeadDim;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int row = blockIdx.x * 4 + wave;
  const int kv = blockIdx.y;
  if (row >= rows_total) return;  // whole wave; the kernel has no barriers
  int b, t;
  prefill_row_position(row, cu_q, cu_k, batch, b, t);
  const int len = cu_k[b + 1] - cu_k[b];
  const int cbase = cu_c[b];
  const int nc = cu_c[b + 1] - cbase;
  const int nvis = t >= kKernel - 1 ? min(nc, (t - (kKernel - 1)) / kStride + 1) : 0;
  const size_t head0 = (size_t(row) * kv_heads + kv) * G;  // first head of the group
  uint4 qb[4];
  load_q<G>(q + head0 * D, qb);
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = kc + size_t(cbase) * rs + size_t(kv) * D;
  const bf16_t* vb = vc + size_t(cbase) * rs + size_t(kv) * D;
  const int cmax = max(nvis - 1, 0);

  if constexpr (!PROBS) {
    float m_run = -INFINITY, l_run = 0.f;
    for (int w0 = 0; w0 < nvis; w0 += 16) {
      KeyTile T;
      load_tile<false>(kb, vb, rs, w0, cmax, T);
      const f32x4_t s = tile_scores(T, qb);
      float sv[4], mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = w0 + 4 * r4 + e < nvis ? s[e] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[e]);
      }
      mx = rows_max(mx);
      if (mx > m_run) {
        l_run *= fast_exp2(m_run - mx);
        m_run = mx;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) l_run += sv[e] == -INFINITY ? 0.f : fast_exp2(sv[e] - m_run);
    }
    l_run = rows_sum(l_run);
    if (r4 == 0 && c16 < G) lse2[head0 + c16] = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
  } else {
    const float lh = lse2[head0 + min(c16, G - 1)];
    f32x4_t acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nb = (len + kBlock - 1) / kBlock;
    float* bs_row = block_scores != nullptr ? block_scores + (size_t(row) * kv_heads + kv) * nb_max : nullptr;
    float carry = 0.f;  // group score of window 16u - 1 (the previous tile's last)
    for (int w0 = 0; w0 < nvis; w0 += 16) {
      KeyTile T;
      load_tile<true>(kb, vb, rs, w0, cmax, T);
      const f32x4_t s = tile_scores(T, qb);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[e] = (c16 < G && w0 + 4 * r4 + e < nvis) ? fast_exp2(s[e] * scale_log2 - lh) : 0.f;
      tile_pv(T, p, acc);
      if (bs_row != nullptr) {
        // group scores of windows w0 + 4 r4 + e, then block w0/4 + r4 over its
        // windows 4i-1 .. 4i+3 (the first one ends the previous lane row)
        float pg[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pg[e] = row_reduce(p[e], OpSum());
        const float up = __shfl(pg[3], (lane + 48) & 63);  // row r4 - 1
        const float first = r4 == 0 ? carry : up;
        const float sc = fmaxf(fmaxf(first, pg[0]), fmaxf(fmaxf(pg[1], pg[2]), pg[3]));
        const int blk = w0 / 4 + r4;
        if (c16 == 0 && blk < nb) bs_row[blk] = sc;
        carry = __shfl(pg[3], 48);
      }
    }
    store_rows<G>(o_cmp, out_f32, head0, acc, 1.f);
    if (lse_nat != nullptr && r4 == 0 && c16 < G) lse_nat[head0 + c16] = lh * kLn2;
    if (bs_row != nullptr) {
      // blocks past the last tile: the first still sees window 16U - 1
      const int first_blk = nvis > 0 ? ((nvis + 15) / 16) * 4 : 0;
      for (int i = first_blk + lane; i < nb_max; i += kWave)
        bs_row[i] = (i == first_blk && nvis > 0 && i < nb) ? carry : 0.f;
    }
  }
}

// --------------------------------------------------------------- window branch

// Sliding-window attention over keys max(0, t-W+1) .. t; with GATED the output
// is g0 * o_cmp + g1 * o_sel + g2 * o_win (the branch outputs are fp32 rows).
template <int G, bool GATED>
__global__ __launch_bounds__(256) void window_prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int rows_total,
    int kv_heads, int window, float scale_log2, void* __restrict__ out, int out_f32,
    float* __restrict__ lse_nat, const float* __restrict__ gates,
    const float* __restrict__ o_cmp, const float* __restrict__ o_sel) {
  constexpr int D = kHeadDim;
  constexpr float kLazy = 8.f;  // log2-domain slack before the running max is raised
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int row = blockIdx.x * 4 + wave;
  const int kv = blockIdx.y;
  if (row >= rows_total) return;  // whole wave; the kernel has no barriers
  int b, t;
  prefill_row_position(row, cu_q, cu_k, batch, b, t);
  const size_t head0 = (size_t(row) * kv_heads + kv) * G;
  uint4 qb[4];
  load_q<G>(q + head0 * D, qb);
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = k + size_t(cu_k[b]) * rs + size_t(kv) * D;
  const bf16_t* vb = v + size_t(cu_k[b]) * rs + size_t(kv) * D;
  const int j_lo = max(0, t - window + 1);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  KeyTile A, B;
  auto step = [&](int key0, const KeyTile& T) {
    const f32x4_t s = tile_scores(T, qb);
    float sv[4], mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = key0 + 4 * r4 + e <= t ? s[e] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = rows_max(mx);
    if (mx > m_run + kLazy) {  // also true for the first tile with a key
      const float alpha = fast_exp2(m_run - mx);
      m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = sv[e] == -INFINITY ? 0.f : fast_exp2(sv[e] - m_run);
      l_run += p[e];
    }
    tile_pv(T, p, acc);
  };
  // double-buffered: the next tile's loads are in flight during this tile's math
  if (t >= 0) load_tile<true>(kb, vb, rs, j_lo, t, A);
  for (int key0 = j_lo; key0 <= t; key0 += 32) {
    const bool has1 = key0 + 16 <= t;
    if (has1) load_tile<true>(kb, vb, rs, key0 + 16, t, B);
    step(key0, A);
    if (has1) {
      if (key0 + 32 <= t) load_tile<true>(kb, vb, rs, key0 + 32, t, A);
      step(key0 + 16, B);
    }
  }
  l_run = rows_sum(l_run);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if constexpr (GATED) {
    if (c16 < G) {
      const size_t h = head0 + c16;
      const float g0 = gates[h * 3 + 0], g1 = gates[h * 3 + 1], g2 = gates[h * 3 + 2];
      const float* pc = o_cmp + h * D + 4 * r4;
      const float* ps = o_sel + h * D + 4 * r4;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float4 a = *reinterpret_cast<const float4*>(pc + 16 * n);
        const float4 s = *reinterpret_cast<const float4*>(ps + 16 * n);
        acc[n][0] = g0 * a.x + g1 * s.x + g2 * acc[n][0] * inv;
        acc[n][1] = g0 * a.y + g1 * s.y + g2 * acc[n][1] * inv;
        acc[n][2] = g0 * a.z + g1 * s.z + g2 * acc[n][2] * inv;
        acc[n][3] = g0 * a.w + g1 * s.w + g2 * acc[n][3] * inv;
      }
    }
    store_rows<G>(out, out_f32, head0, acc, 1.f);
  } else {
    store_rows<G>(out, out_f32, head0, acc, inv);
  }
  if (lse_nat != nullptr && r4 == 0 && c16 < G)
    lse_nat[head0 + c16] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
}

// --------------------------------------------------------------------------- host

template <int G>
static hipError_t launch_cmp_g(const CompressedPrefillArgs& a, hipStream_t s) {
  const dim3 grid((a.rows_total + 3) / 4, a.kv_heads);
  hipError_t e = launch_kernel(
      kKindCmpLse, compressed_prefill_kernel<G, false>, grid, dim3(256), s, a.q, a.kc, a.vc,
      a.cu_q, a.cu_k, a.cu_c, a.batch, a.rows_total, a.kv_heads, a.scale_log2, a.lse2,
      static_cast<void*>(nullptr), 0, static_cast<float*>(nullptr), static_cast<float*>(nullptr),
      0);
  if (e != hipSuccess) return e;
  return launch_kernel(kKindCmpProbs, compressed_prefill_kernel<G, true>, grid, dim3(256), s,
                       a.q, a.kc, a.vc, a.cu_q, a.cu_k, a.cu_c, a.batch, a.rows_total,
                       a.kv_heads, a.scale_log2, a.lse2, a.o_cmp, a.out_f32, a.lse_nat,
                       a.block_scores, a.nb_max);
}

hipError_t launch_compressed_prefill(const CompressedPrefillArgs& a, hipStream_t s) {
  if (a.rows_total == 0) return hipSuccess;
  switch (a.heads / a.kv_heads) {
    case 1: return launch_cmp_g<1>(a, s);
    case 2: return launch_cmp_g<2>(a, s);
    case 4: return launch_cmp_g<4>(a, s);
    case 8: return launch_cmp_g<8>(a, s);
    case 16: return launch_cmp_g<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
static hipError_t launch_win_g(const WindowPrefillArgs& a, hipStream_t s) {
  const dim3 grid((a.rows_total + 3) / 4, a.kv_heads);
  if (a.gates != nullptr)
    return launch_kernel(kKindWindow, window_prefill_kernel<G, true>, grid, dim3(256), s, a.q,
                         a.k, a.v, a.cu_q, a.cu_k, a.batch, a.rows_total, a.kv_heads, a.window,
                         a.scale_log2, a.out, a.out_f32, a.lse_nat, a.gates, a.o_cmp, a.o_sel);
  return launch_kernel(kKindWindow, window_prefill_kernel<G, false>, grid, dim3(256), s, a.q, a.k,
                       a.v, a.cu_q, a.cu_k, a.batch, a.rows_total, a.kv_heads, a.window,
                       a.scale_log2, a.out, a.out_f32, a.lse_nat,
                       static_cast<const float*>(nullptr), static_cast<const float*>(nullptr),
                       static_cast<const float*>(nullptr));
}

hipError_t launch_window_prefill(const WindowPrefillArgs& a, hipStream_t s) {
  if (a.rows_total == 0) return hipSuccess;
  switch (a.heads / a.kv_heads) {
    case 1: return launch_win_g<1>(a, s);
    case 2: return launch_win_g<2>(a, s);
    case 4: return launch_win_g<4>(a, s);
    case 8: return launch_win_g<8>(a, s);
    case 16: return launch_win_g<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nsa
