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
// Design (gfx950): one wave per 4 consecutive query tokens of one sequence and
// KV group; for each token the group's G <= 16 query heads are the 16 columns
// of the MFMA tiles, keys (or windows) go 16 at a time as the rows:
// S^T = K Q^T with four v_mfma_f32_16x16x32_bf16 (Q^T kept in registers), then
// O^T += V^T P^T with eight v_mfma_f32_16x16x32_bf16 (P^T is already in the
// operand layout).  A workgroup holds 4 waves = 16 consecutive tokens; it
// stages each 32-key tile (keys and transposed values, 16 KB) in LDS once, all
// 256 threads loading it, double-buffered so the next tile is in flight while
// the current one is computed, and every wave reads its MFMA operands from
// there.  A tile is thus fetched once per 16 tokens instead of once per wave,
// which is what bounded these kernels (they are limited by operand fetch, not
// by the matrix cores).  The compressed branch runs in two passes: the first
// finds each head's log2 normaliser, the second forms normalised
// probabilities, which give o_cmp directly and, summed over the 16 head
// columns with DPP, the window scores of the group.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ transposed values

// X [N, kv_heads, 128] packed by cu -> XT [batch][kv_heads][128][ld]: one row per
// (sequence, KV head, dim) holding that dim of every token, zero past the
// sequence.  ld is a multiple of 64.  Grid (ld / 64, kv heads, sequences); each
// workgroup moves a 64-token x 128-dim tile through LDS.
__global__ __launch_bounds__(256) void transpose_values_kernel(const bf16_t* __restrict__ x,
                                                               const int* __restrict__ cu,
                                                               int kv_heads, int ld,
                                                               bf16_t* __restrict__ xt) {
  constexpr int D = kHeadDim;
  __shared__ uint16_t tile[64][D + 8];  // rows padded to spread the column reads over banks
  const int tid = threadIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tok0 = blockIdx.x * 64;
  const int start = cu[b], len = cu[b + 1] - start;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i, r = idx >> 4, c = idx & 15;
    const int tok = min(tok0 + r, max(len - 1, 0));
    v[i] = len > 0 ? ld16(x + (size_t(start + tok) * kv_heads + kv) * D + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    if (tok0 + r >= len) v[i] = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i, r = idx >> 4, c = idx & 15;
    *reinterpret_cast<uint4*>(&tile[r][8 * c]) = v[i];
  }
  __syncthreads();
  bf16_t* dst = xt + (size_t(b) * kv_heads + kv) * D * size_t(ld) + tok0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i, d = idx >> 3, tc = idx & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = uint32_t(tile[8 * tc + 2 * e][d]) | (uint32_t(tile[8 * tc + 2 * e + 1][d]) << 16);
    *reinterpret_cast<uint4*>(dst + size_t(d) * ld + 8 * tc) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ------------------------------------------------------------------- key tiles

// One 32-key tile (keys key0 .. key0+31, key0 a multiple of 32) as MFMA operands:
// ka[h] (KeyFrag): A operand of S^T = K Q^T for keys key0 + 16h + c16, dims 32i + 8 r4 .. +8.
// read_val(n): A operand of O^T = V^T P^T for dim 16n + c16; k-slot e < 4
//        holds key key0 + 4 r4 + e, e >= 4 key key0 + 16 + 4 r4 + e - 4 (the same
//        slots the S^T accumulators give P^T).
typedef uint4 KeyFrag[2][4];

// LDS staging of one workgroup's tiles, double-buffered.  Key rows are 256 B
// with their sixteen 16-byte chunks XOR-swizzled by the row's low four bits,
// so the 16 rows one A operand reads hit distinct banks (padding the rows
// instead measured bank conflicts on these reads).  Value rows are 64 B (one
// dim, the tile's 32 keys) in k-slot order: chunk r holds keys 4r..4r+3 then
// 16+4r..16+4r+3, so each value operand is one 16-byte read, and chunk r of
// row d sits at place r ^ ((d >> 1) & 3).  Measured on gfx950 (bank-conflict
// counters over each access pattern alone), that swizzle keeps both the
// operand reads (16 rows, one chunk each) and the 8-byte staging writes
// conflict-free; rows padded to 80 B instead made every operand read take
// two passes.
constexpr int kKRow = kHeadDim;  // bf16 per staged key row (16-byte chunks XOR-swizzled by row)
constexpr int kVRow = 32;        // bf16 per staged value row (4 chunks, swizzled by row)
__device__ __forceinline__ int val_place(int row, int chunk) {
  return row * kVRow + 8 * (chunk ^ ((row >> 1) & 3));
}
struct TileLds {
  bf16_t k[2][32 * kKRow];
  bf16_t v[2][kHeadDim * kVRow];
};

// A tile in flight: with THREADS threads, thread tid holds key chunks
// c = tid + THREADS u (row c / 16, dims 8 (c % 16) .. +8) and value chunks
// c = tid + THREADS u (dim c / 4, keys 8 (c % 4) .. +8) of the 512 16-byte
// chunks of each.
template <int THREADS>
struct TileRegs {
  static constexpr int kPer = 512 / THREADS;
  uint4 k[kPer], v[kPer];
};

// Key rows are clamped to kmax so every load is in bounds (the scores of such
// rows are masked).  Value rows come from the transposed copy, which holds
// zeros past the sequence up to its padded length ldv (a multiple of 64).
template <bool WITH_V, int THREADS>
__device__ __forceinline__ void fetch_tile(const bf16_t* __restrict__ kb, size_t rs,
                                           const bf16_t* __restrict__ vt, int ldv, int key0,
                                           int kmax, TileRegs<THREADS>& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < TileRegs<THREADS>::kPer; ++u) {
    const int c = tid + THREADS * u;
    r.k[u] = ld16(kb + size_t(min(key0 + (c >> 4), kmax)) * rs + 8 * (c & 15));
    if constexpr (WITH_V) r.v[u] = ld16(vt + size_t(c >> 2) * ldv + key0 + 8 * (c & 3));
  }
}

template <bool WITH_V, int THREADS>
__device__ __forceinline__ void stash_tile(TileLds& T, int buf, const TileRegs<THREADS>& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < TileRegs<THREADS>::kPer; ++u) {
    const int c = tid + THREADS * u;
    *reinterpret_cast<uint4*>(&T.k[buf][(c >> 4) * kKRow + 8 * ((c & 15) ^ ((c >> 4) & 15))]) = r.k[u];
    if constexpr (WITH_V) {
      // keys 8kc .. 8kc+3 go to chunk r, keys 8kc+4 .. 8kc+7 to chunk r + 1,
      // both in the chunks' first half (kc < 2) or second half
      const int kc = c & 3, row = c >> 2;
      const int ch = kc < 2 ? 2 * kc : 2 * (kc - 2), half = kc < 2 ? 0 : 4;
      *reinterpret_cast<uint2*>(&T.v[buf][val_place(row, ch) + half]) = make_uint2(r.v[u].x, r.v[u].y);
      *reinterpret_cast<uint2*>(&T.v[buf][val_place(row, ch + 1) + half]) = make_uint2(r.v[u].z, r.v[u].w);
    }
  }
}

__device__ __forceinline__ void read_keys(const TileLds& T, int buf, KeyFrag& ka) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ka[h][i] = *reinterpret_cast<const uint4*>(&T.k[buf][(16 * h + c16) * kKRow + 8 * ((4 * i + r4) ^ c16)]);
}

// ValFrag entry n of a staged value tile (vs: one buffer of TileLds::v).
__device__ __forceinline__ uint4 read_val(const bf16_t* vs, int n) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
  return *reinterpret_cast<const uint4*>(&vs[val_place(16 * n + c16, r4)]);
}

// Tile loop of a workgroup over keys first .. last (first a multiple of 32;
// both the same in every thread).  Every thread takes part in the loads and
// barriers; waves with `active` false (no tokens) skip the compute.  The next
// tile's loads are issued before the current tile is computed and written to
// the other buffer after it; one barrier per tile.
template <bool WITH_V, int THREADS, typename F>
__device__ __forceinline__ void lds_tile_loop(TileLds& T, const bf16_t* __restrict__ kb,
                                              size_t rs, const bf16_t* __restrict__ vt, int ldv,
                                              int first, int last, int kmax, bool active,
                                              F&& process) {
  if (first > last) return;
  TileRegs<THREADS> r;
  fetch_tile<WITH_V>(kb, rs, vt, ldv, first, kmax, r);
  stash_tile<WITH_V>(T, 0, r);
  __syncthreads();
  // one tile from buffer BUF (a constant, so its LDS offsets are immediates)
  auto step = [&](int key0, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    const bool more = key0 + 32 <= last;
    if (more) fetch_tile<WITH_V>(kb, rs, vt, ldv, key0 + 32, kmax, r);
    if (active) {
      KeyFrag ka;
      read_keys(T, BUF, ka);
      process(key0, ka, static_cast<const bf16_t*>(T.v[BUF]));  // values: read_val per fragment
    }
    if (more) stash_tile<WITH_V>(T, BUF ^ 1, r);
    __syncthreads();
  };
  for (int key0 = first; key0 <= last; key0 += 64) {
    step(key0, std::integral_constant<int, 0>());
    if (key0 + 32 > last) break;
    step(key0 + 32, std::integral_constant<int, 1>());
  }
}

// S^T of half h: lane (c16, r4) element e = score of key key0 + 16h + 4 r4 + e
// against head c16.
__device__ __forceinline__ f32x4_t tile_scores(const uint4 (&ka)[2][4], int h, const uint4 (&qb)[4]) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[h][i]),
                                                __builtin_bit_cast(bf16x8_t, qb[i]), s, 0, 0, 0);
  return s;
}

// P^T of one token as the B operand: p[e] in the k-slot order of the value tiles.
__device__ __forceinline__ bf16x8_t pack_p(const float (&p)[8]) {
  return bf16x8_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                  (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
}

// O^T += V^T P^T over the tile's 32 keys for every token of the wave: each value
// fragment is read from LDS once and used by all the tokens.
template <int TPW>
__device__ __forceinline__ void tile_pv(const bf16_t* vs, const bf16x8_t (&pb)[TPW],
                                        f32x4_t (&acc)[TPW][8]) {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const bf16x8_t va = __builtin_bit_cast(bf16x8_t, read_val(vs, n));
#pragma unroll
    for (int j = 0; j < TPW; ++j)
      acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[j], acc[j][n], 0, 0, 0);
  }
}

// Group scores of one 16-window half tile: p[e] is the lane's probability of
// window 4 r4 + e for head c16.  Returns in lane (c16, r4) the sum over the 16
// head columns of window 4 r4 + 2 (c16 & 1) + ((c16 >> 1) & 1); lane 15 of a
// row (c16 & 3 == 3) therefore holds the row's last window.  Pairwise DPP
// exchanges split the four windows over the quad, then two rotations finish
// the sum over the row.
__device__ __forceinline__ float head_sums(const float (&p)[4]) {
  const bool odd = threadIdx.x & 1, hi = (threadIdx.x >> 1) & 1;
  float s0 = odd ? p[2] : p[0], s1 = odd ? p[3] : p[1];
  s0 += dpp<kDppQuadXor1>(odd ? p[0] : p[2]);
  s1 += dpp<kDppQuadXor1>(odd ? p[1] : p[3]);
  float k = hi ? s1 : s0;
  k += dpp<kDppQuadXor2>(hi ? s0 : s1);
  k += dpp<kDppRowRor4>(k);
  return k + dpp<kDppRowRor8>(k);
}

// Value of lane 15 of the previous row (rows 1..3); row 0 gets `first`.
__device__ __forceinline__ float prev_row_last(float x, float first) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(x),
                                                    0x142 /* row_bcast:15 */, 0xE, 0xF, false));
}

// Four bf16 values (two packed words) as floats.
__device__ __forceinline__ float4 bf16x4_to_float4(uint2 w) {
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
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

// Query tokens per workgroup (GT consecutive tokens of one sequence and KV
// group; a template parameter of each kernel); a wave holds TPW of them and a
// workgroup GT / TPW waves.  Fewer tokens per wave means fewer registers and
// more waves per SIMD; the tiles are shared through LDS either way.

// The tokens of one wave: query positions tq0 .. tq0 + n - 1 of sequence b
// (grid z), packed rows row0 .. row0 + n - 1, key positions t0 .. t0 + n - 1.
struct WaveRows {
  int n, row0, t0;
};

// Key positions of the first and last query tokens of workgroup `grp` (GT
// tokens a workgroup) of sequence b; returns false when the workgroup has none.
template <int GT>
__device__ __forceinline__ bool group_span(const int* __restrict__ cu_q,
                                           const int* __restrict__ cu_k, int b, int grp,
                                           int& t_first, int& t_last) {
  const int lq = cu_q[b + 1] - cu_q[b];
  const int lk = cu_k[b + 1] - cu_k[b];
  const int tq = grp * GT;
  if (tq >= lq) return false;
  t_first = tq + (lk - lq);
  t_last = min(tq + GT, lq) - 1 + (lk - lq);
  return true;
}

template <int TPW>
__device__ __forceinline__ WaveRows wave_rows(const int* __restrict__ cu_q,
                                              const int* __restrict__ cu_k, int b, int tile) {
  const int q0 = cu_q[b], lq = cu_q[b + 1] - q0;
  const int lk = cu_k[b + 1] - cu_k[b];
  const int tq = tile * TPW;
  WaveRows r;
  r.n = max(0, min(TPW, lq - tq));
  r.row0 = q0 + tq;
  r.t0 = tq + (lk - lq);
  return r;
}

// PROBS = false: per (row, head) log2 normaliser lse2 = max + log2(sum exp2).
// PROBS = true:  o_cmp, natural-log lse, and the group's block scores.
// vct: the compressed values transposed ([batch][kv][128][ldv]).
template <int G, bool PROBS, int TPW, int GT>
__global__ __launch_bounds__(GT / TPW * kWave)
__attribute__((amdgpu_waves_per_eu(PROBS ? 1 : 3))) void compressed_prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vct,
    int ldv, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    const int* __restrict__ cu_c, int kv_heads, float scale_log2, float* __restrict__ lse2,
    void* __restrict__ o_cmp, int out_f32, float* __restrict__ lse_nat,
    float* __restrict__ block_scores, int nb_max) {
  constexpr int D = kHeadDim;
  __shared__ TileLds T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int kv = blockIdx.y, b = blockIdx.z;
  int t_first, t_last;
  if (!group_span<GT>(cu_q, cu_k, b, blockIdx.x, t_first, t_last)) return;  // whole workgroup
  constexpr int kTpw = TPW, kThreads = GT / TPW * kWave;
  const WaveRows R = wave_rows<TPW>(cu_q, cu_k, b, blockIdx.x * (GT / TPW) + wave);
  const bool active = R.n > 0;  // waves past the sequence only help with the tiles
  const int len = cu_k[b + 1] - cu_k[b];
  const int cbase = cu_c[b];
  const int nc = cu_c[b + 1] - cbase;
  int nvis[kTpw];
  size_t head0[kTpw];  // first head of the group, per token (clamped to a valid row)
  uint4 qb[kTpw][4];
#pragma unroll
  for (int j = 0; j < kTpw; ++j) {
    const int t = R.t0 + j;
    nvis[j] = (j < R.n && t >= kKernel - 1) ? min(nc, (t - (kKernel - 1)) / kStride + 1) : 0;
    head0[j] = (size_t(active ? R.row0 + min(j, R.n - 1) : cu_q[b]) * kv_heads + kv) * G;
    load_q<G>(q + head0[j] * D, qb[j]);
  }
  // windows of the workgroup: those of its last token
  const int nv_wg = t_last >= kKernel - 1 ? min(nc, (t_last - (kKernel - 1)) / kStride + 1) : 0;
  // windows every token of the wave sees (its first token's)
  const int nv_lo = active ? nvis[0] : 0;
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = kc + size_t(cbase) * rs + size_t(kv) * D;
  const bf16_t* vt = vct + (size_t(b) * kv_heads + kv) * D * size_t(ldv);
  const int cmax = max(nv_wg - 1, 0);

  if constexpr (!PROBS) {
    // Each lane keeps its own running maximum and sum over the windows it
    // holds (no cross-lane step per tile); the four lane rows of a head are
    // combined once at the end.  The maximum is raised only when a score
    // passes it by kLazy (log2 domain), so the terms stay below 2^kLazy and
    // most tiles skip the rescale (a branch the whole wave takes or skips).
    constexpr float kLazy = 8.f;
    float m_run[kTpw], l_run[kTpw];
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
      m_run[j] = -INFINITY;
      l_run[j] = 0.f;
    }
    auto process = [&](int w0, const KeyFrag& ka, const bf16_t*) {
      // every token runs every tile (windows past its own count are masked), so
      // the tokens' chains interleave; a tile every token sees whole needs no mask
      const bool inside = w0 + 32 <= nv_lo;
#pragma unroll
      for (int j = 0; j < kTpw; ++j) {
        float sv[8];  // raw scores; the scale goes into the max and the exponent's fma
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t s = tile_scores(ka, h, qb[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[4 * h + e] = s[e];
        }
        if (!inside) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (w0 + 16 * (e >> 2) + 4 * r4 + (e & 3) >= nvis[j]) sv[e] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mx *= scale_log2;
        const bool raise = mx > m_run[j] + kLazy;  // also the lane's first window
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          if (raise) {
            l_run[j] *= fast_exp2(m_run[j] - mx);
            m_run[j] = mx;
          }
        }
        // a lane with no window yet has only masked scores: its terms are 0
        const float mref = m_run[j] == -INFINITY ? 0.f : m_run[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) l_run[j] += fast_exp2(fmaf(sv[e], scale_log2, -mref));
      }
    };
    lds_tile_loop<false, kThreads>(T, kb, rs, vt, ldv, 0, nv_wg - 1, cmax, active, process);
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
      const float m = rows_max(m_run[j]);
      const float l = m == -INFINITY ? 0.f : rows_sum(l_run[j] * fast_exp2(m_run[j] - m));
      if (j < R.n && r4 == 0 && c16 < G)
        lse2[head0[j] + c16] = l > 0.f ? m + __log2f(l) : -INFINITY;
    }
  } else {
    float lh[kTpw], carry[kTpw];
    f32x4_t acc[kTpw][8];
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
        // columns past the group get +inf, so their probabilities are exactly 0
      lh[j] = c16 < G ? lse2[head0[j] + c16] : INFINITY;
      carry[j] = 0.f;  // group score of window w0 - 1 (the previous tile's last)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[j][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int nb = (len + kBlock - 1) / kBlock;
    auto process = [&](int w0, const KeyFrag& ka, const bf16_t* vs) {
      // every token runs every tile (windows past its own count are masked), so
      // the tokens' chains interleave; a tile every token sees whole needs no mask
      const bool inside = w0 + 32 <= nv_lo;
      bf16x8_t pb[kTpw];
#pragma unroll
      for (int j = 0; j < kTpw; ++j) {
        float p[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t s = tile_scores(ka, h, qb[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p[4 * h + e] = fast_exp2(fmaf(s[e], scale_log2, -lh[j]));
        }
        if (!inside) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (w0 + 16 * (e >> 2) + 4 * r4 + (e & 3) >= nvis[j]) p[e] = 0.f;
        }
        pb[j] = pack_p(p);
        if (block_scores != nullptr) {
          // block w0/4 + 4h + r4 covers windows 4i-1 .. 4i+3: the lane row's four
          // windows and the previous row's last (the previous half's last for row 0)
          const float pgA = head_sums({p[0], p[1], p[2], p[3]});
          const float pgB = head_sums({p[4], p[5], p[6], p[7]});
          const float lastA = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pgA), 63));
          const float lastB = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pgB), 63));
          float mA = fmaxf(pgA, dpp<kDppQuadXor1>(pgA));
          mA = fmaxf(mA, dpp<kDppQuadXor2>(mA));
          float mB = fmaxf(pgB, dpp<kDppQuadXor1>(pgB));
          mB = fmaxf(mB, dpp<kDppQuadXor2>(mB));
          const float scA = fmaxf(mA, prev_row_last(pgA, carry[j]));
          const float scB = fmaxf(mB, prev_row_last(pgB, lastA));
          float* bs_row = block_scores + (size_t(R.row0 + j) * kv_heads + kv) * nb_max;
          const int blkA = w0 / 4 + r4, blkB = blkA + 4;
          if (w0 < nvis[j] && c16 == 0) {
            if (blkA < nb) bs_row[blkA] = scA;
            if (blkB < nb) bs_row[blkB] = scB;
          }
          if (w0 < nvis[j]) carry[j] = lastB;                   // window w0 + 31
        }
      }
      tile_pv<kTpw>(vs, pb, acc);
    };
    lds_tile_loop<true, kThreads>(T, kb, rs, vt, ldv, 0, nv_wg - 1, cmax, active, process);
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
      if (j >= R.n) continue;
      store_rows<G>(o_cmp, out_f32, head0[j], acc[j], 1.f);
      if (lse_nat != nullptr && r4 == 0 && c16 < G) lse_nat[head0[j] + c16] = lh[j] * kLn2;
      if (block_scores != nullptr) {
        // blocks past the token's last tile: the first still sees the tile's last
        // window; blocks past the sequence are 0
        float* bs_row = block_scores + (size_t(R.row0 + j) * kv_heads + kv) * nb_max;
        const int first_blk = nvis[j] > 0 ? ((nvis[j] + 31) / 32) * 8 : 0;
        for (int i = min(first_blk, nb) + lane; i < nb_max; i += kWave)
          bs_row[i] = (i == first_blk && nvis[j] > 0 && i < nb) ? carry[j] : 0.f;
      }
    }
  }
}

// --------------------------------------------------------------- window branch

// Sliding-window attention over keys max(0, t-W+1) .. t; with GATED the output
// is g0 * o_cmp + g1 * o_sel + g2 * o_win (the other branches' outputs are bf16 rows;
// o_sel32, when given, holds the selected branch as float32 rows instead).
// The wave's tokens share the key tiles of the union of their windows.
// vtr: the values transposed ([batch][kv][128][ldv]).
template <int G, bool GATED, int TPW, int GT>
__global__ __launch_bounds__(GT / TPW * kWave) void window_prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ vtr,
    int ldv, const int* __restrict__ cu_q, const int* __restrict__ cu_k, int kv_heads,
    int window, float scale_log2, void* __restrict__ out, int out_f32,
    float* __restrict__ lse_nat, const float* __restrict__ gates,
    const bf16_t* __restrict__ o_cmp, const bf16_t* __restrict__ o_sel,
    const float* __restrict__ o_sel32) {
  constexpr int D = kHeadDim;
  constexpr float kLazy = 8.f;  // log2-domain slack before the running max is raised
  __shared__ TileLds T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int kv = blockIdx.y, b = blockIdx.z;
  int t_first, t_last;
  if (!group_span<GT>(cu_q, cu_k, b, blockIdx.x, t_first, t_last)) return;  // whole workgroup
  constexpr int kTpw = TPW, kThreads = GT / TPW * kWave;
  const WaveRows R = wave_rows<TPW>(cu_q, cu_k, b, blockIdx.x * (GT / TPW) + wave);
  const bool active = R.n > 0;  // waves past the sequence only help with the tiles
  size_t head0[kTpw];
  uint4 qb[kTpw][4];
#pragma unroll
  for (int j = 0; j < kTpw; ++j) {
    head0[j] = (size_t(active ? R.row0 + min(j, R.n - 1) : cu_q[b]) * kv_heads + kv) * G;
    load_q<G>(q + head0[j] * D, qb[j]);
  }
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = k + size_t(cu_k[b]) * rs + size_t(kv) * D;
  const bf16_t* vt = vtr + (size_t(b) * kv_heads + kv) * D * size_t(ldv);
  // keys of the workgroup: the union of its tokens' windows, tiles 32-aligned
  const int j_lo = max(0, t_first - window + 1) & ~31;
  float m_run[kTpw], l_run[kTpw];
  f32x4_t acc[kTpw][8];
#pragma unroll
  for (int j = 0; j < kTpw; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[j][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // keys every token of the wave sees: from its last token's window start to
  // its first token
  const int in_lo = R.t0 + R.n - 1 - window + 1, in_hi = R.t0;
  auto process = [&](int key0, const KeyFrag& ka, const bf16_t* vs) {
    // every token runs every tile of the union (keys outside its own window
    // are masked), so the tokens' chains interleave; a tile every token sees
    // whole needs no mask
    const bool inside = key0 >= in_lo && key0 + 31 <= in_hi;
    bf16x8_t pb[kTpw];
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
      const int t = R.t0 + j;
      const int lo = max(0, t - window + 1);
      float sv[8];  // raw scores; the scale goes into the max and the exponent's fma
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t s = tile_scores(ka, h, qb[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * h + e] = s[e];
      }
      if (!inside) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = key0 + 16 * (e >> 2) + 4 * r4 + (e & 3);
          if (key > t || key < lo) sv[e] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = rows_max(mx) * scale_log2;
      if (mx > m_run[j] + kLazy) {  // also true for the first tile with a key
        const float alpha = fast_exp2(m_run[j] - mx);
        m_run[j] = mx;
        l_run[j] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[j][n] *= alpha;
      }
      float p[8];
      if (m_run[j] == -INFINITY) {  // no key of this token yet (same in every lane)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = 0.f;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sv[e], scale_log2, -m_run[j]));
          l_run[j] += p[e];
        }
      }
      pb[j] = pack_p(p);
    }
    tile_pv<kTpw>(vs, pb, acc);
  };
  lds_tile_loop<true, kThreads>(T, kb, rs, vt, ldv, j_lo, t_last, t_last, active, process);
#pragma unroll
  for (int j = 0; j < kTpw; ++j) {
    const float l = rows_sum(l_run[j]);
    if (j >= R.n) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if constexpr (GATED) {
      if (c16 < G) {
        const size_t h = head0[j] + c16;
        const float g0 = gates[h * 3 + 0], g1 = gates[h * 3 + 1], g2 = gates[h * 3 + 2];
        const bf16_t* pc = o_cmp + h * D + 4 * r4;
        const bf16_t* ps = o_sel + h * D + 4 * r4;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float4 a = bf16x4_to_float4(*reinterpret_cast<const uint2*>(pc + 16 * n));
          const float4 s = o_sel32 != nullptr
                               ? *reinterpret_cast<const float4*>(o_sel32 + h * D + 4 * r4 + 16 * n)
                               : bf16x4_to_float4(*reinterpret_cast<const uint2*>(ps + 16 * n));
          acc[j][n][0] = g0 * a.x + g1 * s.x + g2 * acc[j][n][0] * inv;
          acc[j][n][1] = g0 * a.y + g1 * s.y + g2 * acc[j][n][1] * inv;
          acc[j][n][2] = g0 * a.z + g1 * s.z + g2 * acc[j][n][2] * inv;
          acc[j][n][3] = g0 * a.w + g1 * s.w + g2 * acc[j][n][3] * inv;
        }
      }
      store_rows<G>(out, out_f32, head0[j], acc[j], 1.f);
    } else {
      store_rows<G>(out, out_f32, head0[j], acc[j], inv);
    }
    if (lse_nat != nullptr && r4 == 0 && c16 < G)
      lse_nat[head0[j] + c16] = l > 0.f ? (m_run[j] + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------ block-mask attention

// Block-sparse attention with a block mask (TileLang NSA, section 1): query
// block i of sequence b and head h attends to the keys of every key block j
// with mask[b][h][i][j] != 0 (and, when causal, to keys <= its own position).
// Multi-head: Q, K, V [N, heads, 128] packed by cu_seqlens (queries are the
// sequence's own tokens).  One workgroup per (query block of 64 tokens, head,
// sequence); each of its 4 waves holds one column tile of 16 tokens (the MFMA
// columns are tokens of one head here; 4 waves of one tile measured 10-15%
// faster than 2 waves of two).  The active key blocks are listed in LDS from
// the mask row (16-bit ids, so four workgroups fit a CU's LDS), and their
// 32-key tiles staged and consumed as in the window branch.
constexpr int kMaskWaves = 4, kMaskTpw = 1, kMaskThreads = kMaskWaves * kWave;
constexpr int kMaskMaxBlocks = kBlockMaskMaxLen / 64;
static_assert(kMaskWaves * kMaskTpw * 16 == 64, "a workgroup covers one 64-token query block");

template <bool CAUSAL>
__global__ __launch_bounds__(kMaskThreads) __attribute__((amdgpu_waves_per_eu(2))) void blockmask_attn_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ vtr,
    int ldv, const unsigned char* __restrict__ mask, int nb_max, const int* __restrict__ cu,
    int heads, float scale_log2, bf16_t* __restrict__ out) {
  constexpr int D = kHeadDim;
  constexpr float kLazy = 8.f;
  __shared__ TileLds T;
  __shared__ unsigned short blocks_s[kMaskMaxBlocks];
  __shared__ int n_tiles_s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int s0 = cu[b], L = cu[b + 1] - s0;
  if (64 * qb >= L) return;  // whole workgroup
  const int nkb = min((L + 63) / 64, nb_max);  // a max_seqlen below L reads no mask past nb_max
  // active key tiles of this query block, ascending (wave 0 scans the mask row)
  if (wave == 0) {
    const unsigned char* mrow = mask + ((size_t(b) * heads + h) * nb_max + qb) * nb_max;
    int base = 0;
    for (int j0 = 0; j0 < nkb; j0 += kWave) {
      const int j = j0 + lane;
      const bool on = j < nkb && mrow[j] != 0 && (!CAUSAL || j <= qb);
      const unsigned long long m = __ballot(on);
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (on) blocks_s[pos] = static_cast<unsigned short>(j);
      base += __popcll(m);
    }
    if (lane == 0) n_tiles_s = 2 * base;
  }
  // the wave's tokens: 64 qb + 16 (kMaskTpw wave + jt) + c16 (jt < kMaskTpw)
  int tok[kMaskTpw];
  uint4 qbop[kMaskTpw][4];
#pragma unroll
  for (int jt = 0; jt < kMaskTpw; ++jt) {
    tok[jt] = 64 * qb + 16 * (kMaskTpw * wave + jt) + c16;
    const bf16_t* qp = q + (size_t(s0 + min(tok[jt], L - 1)) * heads + h) * D + 8 * r4;
#pragma unroll
    for (int i = 0; i < 4; ++i) qbop[jt][i] = ld16(qp + 32 * i);
  }
  float m_run[kMaskTpw], l_run[kMaskTpw];
  f32x4_t acc[kMaskTpw][8];
#pragma unroll
  for (int jt = 0; jt < kMaskTpw; ++jt) {
    m_run[jt] = -INFINITY;
    l_run[jt] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[jt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const int n_tiles = n_tiles_s;
  const size_t rs = size_t(heads) * D;
  const bf16_t* kb = k + size_t(s0) * rs + size_t(h) * D;
  const bf16_t* vt = vtr + (size_t(b) * heads + h) * D * size_t(ldv);
  auto process = [&](int key0, const KeyFrag& ka, const bf16_t* vs) {
    // keys past the sequence, and (causal) keys after a token, are masked; a
    // tile wholly before the query block and inside the sequence needs no mask
    const bool inside = key0 + 31 < L && (!CAUSAL || key0 + 31 < 64 * qb);
    bf16x8_t pb[kMaskTpw];
#pragma unroll
    for (int jt = 0; jt < kMaskTpw; ++jt) {
      float sv[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4_t sc = tile_scores(ka, hh, qbop[jt]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * hh + e] = sc[e];
      }
      if (!inside) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = key0 + 16 * (e >> 2) + 4 * r4 + (e & 3);
          if (key >= L || (CAUSAL && key > tok[jt])) sv[e] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = rows_max(mx) * scale_log2;
      if (mx > m_run[jt] + kLazy) {
        const float alpha = fast_exp2(m_run[jt] - mx);
        m_run[jt] = mx;
        l_run[jt] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[jt][n] *= alpha;
      }
      float p[8];
      if (m_run[jt] == -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = 0.f;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sv[e], scale_log2, -m_run[jt]));
          l_run[jt] += p[e];
        }
      }
      pb[jt] = pack_p(p);
    }
    tile_pv<kMaskTpw>(vs, pb, acc);
  };
  // the listed tiles, double-buffered through LDS as in lds_tile_loop
  if (n_tiles > 0) {
    TileRegs<kMaskThreads> r;
    auto tile_key0 = [&](int it) { return 64 * int(blocks_s[it >> 1]) + 32 * (it & 1); };
    fetch_tile<true>(kb, rs, vt, ldv, tile_key0(0), L - 1, r);
    stash_tile<true>(T, 0, r);
    __syncthreads();
    // unrolled by the two buffers, so their LDS offsets are immediates
    auto step = [&](int it, auto buf_c) {
      constexpr int BUF = decltype(buf_c)::value;
      const bool more = it + 1 < n_tiles;
      if (more) fetch_tile<true>(kb, rs, vt, ldv, tile_key0(it + 1), L - 1, r);
      KeyFrag ka;
      read_keys(T, BUF, ka);
      process(tile_key0(it), ka, static_cast<const bf16_t*>(T.v[BUF]));
      if (more) stash_tile<true>(T, BUF ^ 1, r);
      __syncthreads();
    };
    for (int it = 0; it < n_tiles; it += 2) {
      step(it, std::integral_constant<int, 0>());
      if (it + 1 >= n_tiles) break;
      step(it + 1, std::integral_constant<int, 1>());
    }
  }
#pragma unroll
  for (int jt = 0; jt < kMaskTpw; ++jt) {
    const float l = rows_sum(l_run[jt]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (tok[jt] >= L) continue;
    bf16_t* dst = out + (size_t(s0 + tok[jt]) * heads + h) * D + 4 * r4;
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<uint2*>(dst + 16 * n) =
          make_uint2(pack_bf16x2(acc[jt][n][0] * inv, acc[jt][n][1] * inv),
                     pack_bf16x2(acc[jt][n][2] * inv, acc[jt][n][3] * inv));
  }
}

// --------------------------------------------------------------------------- host

// Tokens per wave and per workgroup of each kernel: the normaliser pass keeps
// no output accumulators and holds 4 tokens a wave, 16 a workgroup; the passes
// with P.V hold 1 a wave, 8 a workgroup (about 100 VGPRs, four waves per SIMD:
// 6% faster than 2 a wave and 16 a workgroup at 190 VGPRs, while the normaliser
// pass measured 23% slower at 8 a workgroup).
constexpr int kTpwLse = 4, kGtLse = 16, kTpwOut = 1, kGtOut = 8;

// Grid: (groups of gt tokens, kv head, sequence).
static dim3 prefill_grid(int max_seqlen_q, int kv_heads, int batch, int gt) {
  return dim3((max_seqlen_q + gt - 1) / gt, kv_heads, batch);
}

static dim3 prefill_block(int tpw, int gt) { return dim3(gt / tpw * kWave); }

int transposed_ld(int max_len) { return (max_len + 63) / 64 * 64; }

size_t transposed_bytes(int batch, int kv_heads, int max_len) {
  return size_t(batch) * kv_heads * kHeadDim * size_t(transposed_ld(max_len)) * sizeof(bf16_t);
}

static hipError_t launch_transpose(const bf16_t* x, const int* cu, int batch, int kv_heads,
                                   int max_len, bf16_t* xt, hipStream_t s) {
  const int ld = transposed_ld(max_len);
  if (ld == 0 || batch == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_values_kernel, dim3(ld / 64, kv_heads, batch), dim3(256), 0, s, x,
                     cu, kv_heads, ld, xt);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_cmp_g(const CompressedPrefillArgs& a, hipStream_t s) {
  const int ldv = transposed_ld(a.max_windows);
  hipError_t e = launch_transpose(a.vc, a.cu_c, a.batch, a.kv_heads, a.max_windows, a.vct, s);
  if (e != hipSuccess) return e;
  e = launch_kernel(kKindCmpLse, compressed_prefill_kernel<G, false, kTpwLse, kGtLse>,
                    prefill_grid(a.max_seqlen_q, a.kv_heads, a.batch, kGtLse),
                    prefill_block(kTpwLse, kGtLse), s, a.q,
                    a.kc, static_cast<const bf16_t*>(a.vct), ldv, a.cu_q, a.cu_k, a.cu_c,
                    a.kv_heads, a.scale_log2, a.lse2, static_cast<void*>(nullptr), 0,
                    static_cast<float*>(nullptr), static_cast<float*>(nullptr), 0);
  if (e != hipSuccess) return e;
  return launch_kernel(kKindCmpProbs, compressed_prefill_kernel<G, true, kTpwOut, kGtOut>,
                       prefill_grid(a.max_seqlen_q, a.kv_heads, a.batch, kGtOut),
                       prefill_block(kTpwOut, kGtOut), s,
                       a.q, a.kc, static_cast<const bf16_t*>(a.vct), ldv, a.cu_q, a.cu_k, a.cu_c,
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
  const dim3 grid = prefill_grid(a.max_seqlen_q, a.kv_heads, a.batch, kGtOut);
  const int ldv = transposed_ld(a.max_seqlen_k);
  hipError_t e = launch_transpose(a.v, a.cu_k, a.batch, a.kv_heads, a.max_seqlen_k, a.vt, s);
  if (e != hipSuccess) return e;
  const bf16_t* vt = a.vt;
  if (a.gates != nullptr)
    return launch_kernel(kKindWindow, window_prefill_kernel<G, true, kTpwOut, kGtOut>, grid,
                         prefill_block(kTpwOut, kGtOut), s, a.q,
                         a.k, vt, ldv, a.cu_q, a.cu_k, a.kv_heads, a.window, a.scale_log2, a.out,
                         a.out_f32, a.lse_nat, a.gates, a.o_cmp, a.o_sel, a.o_sel32);
  return launch_kernel(kKindWindow, window_prefill_kernel<G, false, kTpwOut, kGtOut>, grid,
                       prefill_block(kTpwOut, kGtOut), s, a.q, a.k,
                       vt, ldv, a.cu_q, a.cu_k, a.kv_heads, a.window, a.scale_log2, a.out,
                       a.out_f32, a.lse_nat, static_cast<const float*>(nullptr),
                       static_cast<const bf16_t*>(nullptr), static_cast<const bf16_t*>(nullptr),
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

hipError_t launch_blockmask_attn(const bf16_t* q, const bf16_t* k, const bf16_t* v,
                                 const unsigned char* mask, int causal, bf16_t* out,
                                 const int* cu, int batch, int max_seqlen, int heads,
                                 float scale_log2, bf16_t* vt, hipStream_t s) {
  if (batch == 0 || max_seqlen == 0) return hipSuccess;
  hipError_t e = launch_transpose(v, cu, batch, heads, max_seqlen, vt, s);
  if (e != hipSuccess) return e;
  const int nb = (max_seqlen + 63) / 64;
  const int ldv = transposed_ld(max_seqlen);
  auto kern = causal ? blockmask_attn_kernel<true> : blockmask_attn_kernel<false>;
  return launch_kernel(kKindMask, kern, dim3(nb, heads, batch), dim3(kMaskThreads), s, q, k,
                       static_cast<const bf16_t*>(vt), ldv, mask, nb, cu, heads, scale_log2, out);
}

}  // namespace nsa
