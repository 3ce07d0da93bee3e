// Compressed-key scoring and top-k block selection.
//
// What is computed (NOSA-1B core components, component 3 stage 1; NOSA-1B source
// analysis part 3, "beyond the kernel"): for the newest token of a sequence and
// each query head h, softmax over the visible compressed windows of
// scale * q_h . K_c[c]; the probabilities summed over the GQA group; max-pooled
// onto 64-token blocks (windows 4i-1 .. 4i+3 overlap block i for windows of 32
// with stride 16); plus w * the same max of the pooled CIS; then the init and
// local blocks forced in and the best other blocks picked, ids ascending.
//
// window_logits_kernel -- one-dimensional grid over (sequence, kv head, chunk of
//   64 windows) in XCD-grouped order, 4 waves of 16 windows, on the matrix
//   cores: S^T = Kc Q^T with the compressed-key rows loaded straight into the A
//   operand and the group's queries as the B operand
//   (four v_mfma_f32_16x16x32_bf16 per wave when both are bf16, else thirty-two
//   v_mfma_f32_16x16x4_f32 in full fp32).  Each compressed key is read from HBM
//   once for the whole GQA group.
//   Outputs: per window and head exp2(logit - chunk max) (log2-domain logits), the
//   per-chunk (max, sum of exp2) per head, and the
//   CIS maximum of the blocks the chunk owns (blocks 16j..16j+15, the last chunk
//   also block 16*n_chunks).  The workgroup owning the newest window can first
//   recompute that window of the K_c and pooled-CIS caches (decode refresh).
// select_kernel -- one workgroup of 512 threads per (row, kv head), for rows
//   with more blocks than the single-kernel decode path takes (up to 4096).
//   Derives the block scores (group probabilities of the windows, from the
//   logits kernel's per-chunk normalisers) or reads given scores, then selects
//   with the histogram top-k of select_core.h: forced blocks, and among the
//   others a 256-bin histogram of order-preserving keys over their range locates
//   the bin holding the k-th best; higher bins are taken, lower bins dropped;
//   a boundary bin of at most 64 candidates is ranked exactly by (score desc,
//   id asc), a larger one refined on the next 8 bits.  Chosen ids are written in
//   ascending order from wave ballots and one scan of the per-(slab, wave)
//   counts.
// select_wave_kernel -- one wave per (row, kv head) for many short rows (prefill).
// Every load phase is branch-free (indices clamped into range, values masked)
// so all of a thread's loads are in flight together.  No kernel waits on another
// workgroup: each hand-off is a kernel boundary.
#include "common.h"
#include "launch.h"
#include "select_core.h"

namespace nsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void row_position(int row, const int* __restrict__ cu_q,
                                             const int* __restrict__ cu_k, int batch, int& b,
                                             int& t) {
  if (cu_q == nullptr) {
    b = row;
    t = cu_k[b + 1] - cu_k[b] - 1;
    return;
  }
  int lo = 0, hi = batch - 1;  // last sequence whose first row is <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  b = lo;
  t = (row - cu_q[b]) + ((cu_k[b + 1] - cu_k[b]) - (cu_q[b + 1] - cu_q[b]));
}

// ------------------------------------------------------------ kernel 1: logits

constexpr int kCisSpan = kChunkWindows + 5;  // windows c0-1 .. c0+67 (17 owned blocks)

template <int G, typename TQ, typename TKC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void window_logits_kernel(
    const TQ* __restrict__ q, TKC* __restrict__ kc, const int* __restrict__ cu_k,
    const int* __restrict__ cu_c, float* __restrict__ logits, float2* __restrict__ part,
    float* __restrict__ cisb, float* __restrict__ cis_pooled, int kv_heads, int ldc,
    int n_chunk_max, int ldb, float scale_log2, const TQ* __restrict__ k_src,
    const float* __restrict__ cis_src) {
  // bf16 queries and keys: 16x16x32 bf16 tiles; an fp32 operand: 16x16x4 fp32 tiles
  constexpr bool kBf16 = sizeof(TQ) == 2 && sizeof(TKC) == 2;
  constexpr int D = kHeadDim;
  __shared__ uint32_t new_s[D / 2];  // refreshed compressed key, bf16 pairs
  __shared__ float newf_s[D];        // refreshed compressed key as the cache holds it
  __shared__ float cisw_s[kCisSpan];
  __shared__ float red_s[2][4][16];
  // one-dimensional grid over (sequence, kv head, chunk): the chunks of one
  // (sequence, kv head) run on one XCD, the one its decode splits run on
  const int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  const int unit_i = m / n_chunk_max;
  const int chunk = m - unit_i * n_chunk_max, kv = unit_i % kv_heads, b = unit_i / kv_heads;
  const int start = cu_k[b];
  const int len = cu_k[b + 1] - start;
  const int cbase = cu_c[b];
  const int nc = cu_c[b + 1] - cbase;
  const int nvis = min(nc, full_windows_dev(len));  // decode query at t = len-1
  const int c0 = chunk * kChunkWindows;
  if (c0 >= nvis) return;
  const int n_chunk = (nvis + kChunkWindows - 1) / kChunkWindows;
  const int nb = (len + kBlock - 1) / kBlock;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const size_t unit = size_t(b) * kv_heads + kv;
  // the newest window, recomputed from K in this workgroup (decode append), else -1
  const int rw = (k_src != nullptr && nvis == nc && nc - 1 >= c0 && nc - 1 < c0 + kChunkWindows)
                     ? nc - 1 : -1;

  // ---- every global load of the workgroup, before the first use.  Lane (c16, r4)
  // holds row c16 of the A operand (window ca) and column c16 of the B operand
  // (query head c16; zero past G).  bf16 tiles: dims 32i + 8 r4 .. +8 form the k
  // range of tile i.  fp32 tiles: tile 4i + e takes dim 16i + 4 r4 + e as its k
  // index r4, so the 32 tiles cover every dim once and each load instruction
  // reads 64 contiguous bytes of a row (the four lanes r4 side by side).
  const int ca = c0 + 16 * wave + c16;
  const TKC* krow = kc + (size_t(cbase + min(ca, nvis - 1)) * kv_heads + kv) * D;
  const TQ* qrow = q + (unit * G + min(c16, G - 1)) * D;
  uint4 ka[4], qb[4];
  float kf[32], qf[32];
  if constexpr (kBf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[i] = ld16(krow + 32 * i + 8 * r4);
      qb[i] = ld16(qrow + 32 * i + 8 * r4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load4f(krow + 16 * i + 4 * r4, &kf[4 * i]);
      load4f(qrow + 16 * i + 4 * r4, &qf[4 * i]);
    }
  }
  float cisv = -INFINITY;
  if (cis_pooled != nullptr && tid < kCisSpan) {
    const int cw = c0 - 1 + tid;
    cisv = cis_pooled[(size_t(cbase) + min(max(cw, 0), nvis - 1)) * kv_heads + kv];
    if (cw < 0 || cw >= nvis) cisv = -INFINITY;
  }
  float racc = 0.f, rcis = 0.f;
  if (rw >= 0) {
    const int j0 = start + kStride * rw;
    if (tid < D) {
      float xv[kKernel];
#pragma unroll
      for (int j = 0; j < kKernel; ++j)
        xv[j] = to_f32(k_src[(size_t(j0 + j) * kv_heads + kv) * D + tid]);
      // same summation order as the pooling kernel: each half of the window
      // token by token, then the two halves
      float h0 = 0.f, h1 = 0.f;
#pragma unroll
      for (int j = 0; j < kStride; ++j) h0 += xv[j];
#pragma unroll
      for (int j = kStride; j < kKernel; ++j) h1 += xv[j];
      racc = (h0 + h1) / float(kKernel);
    } else if (cis_src != nullptr && tid >= 128 && tid < 128 + kKernel) {
      rcis = cis_src[size_t(j0 + tid - 128) * kv_heads + kv];
    }
  }

  // ---- refresh of the newest window, CIS of the windows around the chunk
  if (tid < kCisSpan && (rw < 0 || c0 - 1 + tid != rw)) cisw_s[tid] = cisv;
  if (rw >= 0) {
    if (tid < D) {
      TKC st;
      store_f32(&st, racc);
      newf_s[tid] = to_f32(st);  // what a reader of the cache sees
      kc[(size_t(cbase + rw) * kv_heads + kv) * D + tid] = st;
    }
    if (wave == 2) {
      // lanes 0..31 of wave 2 hold the window's 32 scores; summed as the
      // pooling kernel does: each half in token order, then the two halves
      float h0 = 0.f, h1 = 0.f;
#pragma unroll
      for (int j = 0; j < kStride; ++j)
        h0 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rcis), j));
#pragma unroll
      for (int j = kStride; j < kKernel; ++j)
        h1 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rcis), j));
      const float pooled = (h0 + h1) / float(kKernel);
      if (lane == 0 && cis_pooled != nullptr) {
        if (cis_src != nullptr) cis_pooled[size_t(cbase + rw) * kv_heads + kv] = pooled;
        cisw_s[rw - c0 + 1] =
            cis_src != nullptr ? pooled : cis_pooled[size_t(cbase + rw) * kv_heads + kv];
      }
    }
  }
  __syncthreads();
  if constexpr (kBf16) {
    if (rw >= 0) {
      // pack the refreshed row (already bf16-exact) for the lane that owns it
      if (tid < D / 2) new_s[tid] = pack_bf16x2(newf_s[2 * tid], newf_s[2 * tid + 1]);
      __syncthreads();
      if (ca == rw) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ka[i] = *reinterpret_cast<const uint4*>(&new_s[(32 * i + 8 * r4) / 2]);
      }
    }
    if (c16 >= G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qb[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    if (ca == rw) {
#pragma unroll
      for (int j = 0; j < 32; ++j) kf[j] = newf_s[16 * (j >> 2) + 4 * r4 + (j & 3)];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) qf[j] = c16 < G ? qf[j] : 0.f;
  }

  // ---- block CIS maxima of the blocks this chunk owns
  if (cis_pooled != nullptr && tid < 17) {
    const int i = 16 * chunk + tid;
    if ((tid < 16 || chunk == n_chunk - 1) && i < nb) {
      float m = -INFINITY;
#pragma unroll
      for (int e = 0; e < 5; ++e) m = fmaxf(m, cisw_s[4 * tid + e]);
      cisb[unit * ldb + i] = m == -INFINITY ? 0.f : m;
    }
  }

  // ---- S^T = Kc Q^T on the matrix cores, then chunk max and sum of exp2 per head
  f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kBf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[i]),
                                                     __builtin_bit_cast(bf16x8_t, qb[i]), sacc,
                                                     0, 0, 0);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[j], qf[j], sacc, 0, 0, 0);
  }
  // lane (c16, r4): windows cw0 .. cw0+3 of head c16
  float* lrow = logits + unit * G * ldc;
  const int cw0 = c0 + 16 * wave + 4 * r4;
  float sv[4];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sv[e] = cw0 + e < nvis ? sacc[e] * scale_log2 : -INFINITY;
    mx = fmaxf(mx, sv[e]);
  }
  mx = cross32(cross16(mx, OpMax()), OpMax());
  if (r4 == 0) red_s[0][wave][c16] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_s[0][0][c16], red_s[0][1][c16]),
                        fmaxf(red_s[0][2][c16], red_s[0][3][c16]));
  // stored per window: exp2(logit - chunk max), 0 for windows not visible
  float ev[4], l = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ev[e] = sv[e] == -INFINITY ? 0.f : fast_exp2(sv[e] - M);
    l += ev[e];
  }
  if (c16 < G)
    *reinterpret_cast<float4*>(lrow + size_t(c16) * ldc + cw0) = make_float4(ev[0], ev[1], ev[2], ev[3]);
  l = cross32(cross16(l, OpSum()), OpSum());
  if (r4 == 0) red_s[1][wave][c16] = l;
  __syncthreads();
  if (tid < G)
    part[(unit * n_chunk_max + chunk) * G + tid] =
        make_float2(M, red_s[1][0][tid] + red_s[1][1][tid] + red_s[1][2][tid] + red_s[1][3][tid]);
}

// ------------------------------------------------------------ kernel 2: select

constexpr int kSelThreads = 512;
using BigSel = SelCfg<kSelThreads, kMaxSortBlocks>;

template <int G, bool FROM_LOGITS>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ logits, const float2* __restrict__ part,
    const float* __restrict__ cisb, float cis_weight, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, const int* __restrict__ cu_c, int batch,
    float* __restrict__ block_scores, float* __restrict__ window_probs, int kv_heads,
    int nc_max, int ldc, int nb_max, int n_chunk_max, int ldb, int* __restrict__ indices,
    int topk, int n_init, int n_local, int n_cand) {
  __shared__ SelShared<kSelThreads, kMaxSortBlocks> S;
  const int tid = threadIdx.x;
  // one-dimensional grid over (row, kv head) in XCD-grouped order: a decode row
  // is selected on the XCD that wrote its window logits
  const int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  const int row = m / kv_heads, kv = m - row * kv_heads;
  const size_t unit = size_t(m);
  ScoreInputs<G, kSelThreads, kMaxSortBlocks> sin;
  if constexpr (FROM_LOGITS)  // in flight while the row's position is found
    load_score_inputs(sin, logits, part, cisb, unit, n_chunk_max, ldc, ldb);
  int b, t;
  row_position(row, cu_q, cu_k, batch, b, t);
  const int len = cu_k[b + 1] - cu_k[b];
  const int nb = min(nb_max, (len + kBlock - 1) / kBlock);
  float sc[BigSel::kPer], scc[BigSel::kPer];
  if constexpr (FROM_LOGITS) {
    const int nc = cu_c[b + 1] - cu_c[b];
    const int nvis = min(nc, full_windows_dev(len));
    block_scores_from_logits<G, kSelThreads, kMaxSortBlocks>(
        S, sc, scc, n_cand > 0, sin, logits, cisb, cis_weight, unit, nvis, nb, ldc, nb_max,
        nc_max, block_scores, window_probs);
  } else {
    const int n_slab = (nb + kSelThreads - 1) / kSelThreads;  // uniform
#pragma unroll
    for (int u = 0; u < BigSel::kPer; ++u) {
      sc[u] = u < n_slab ? block_scores[unit * nb_max + min(tid + kSelThreads * u, nb - 1)] : 0.f;
      scc[u] = 0.f;
    }
  }
  if (indices == nullptr) return;
  int* out = indices + unit * topk;
  const int total = topk_select<kSelThreads, kMaxSortBlocks>(
      S, sc, scc, n_cand, sel_geometry(t, nb, topk, n_init, n_local, n_cand), topk,
      [&](int pos, int id) { out[pos] = id; });
  for (int i = total + tid; i < topk; i += kSelThreads) out[i] = -1;
}

// ------------------------------------------------- kernel 3: select, one wave per row

// Top-k of given block scores with one wave per (row, kv head), for many short
// rows (prefill): lane l holds ids l + 64j (j < PER) in registers; the free
// places are filled one per round with the best remaining score (ties to the
// lower id) by a wave max and a wave min of the candidate ids.  Same rules and
// output as select_kernel.
template <int PER>
__global__ __launch_bounds__(256) void select_wave_kernel(
    const float* __restrict__ block_scores, int* __restrict__ indices, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int batch, int units, int kv_heads, int nb_max, int topk,
    int n_init, int n_local) {
  static_assert(PER <= 64, "one id bit per slot");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= units) return;  // whole wave; the kernel has no barriers
  int b, t;
  row_position(unit / kv_heads, cu_q, cu_k, batch, b, t);
  const int len = cu_k[b + 1] - cu_k[b];
  const int nb = min(nb_max, (len + kBlock - 1) / kBlock);
  const int n_elig = t >= 0 ? min(nb, t / kBlock + 1) : 0;
  const int f_init = min(n_init, n_elig);
  const int f_loc = max(max(0, n_elig - n_local), f_init);
  const int n_forced = f_init + (n_elig - f_loc);
  const int n_free = n_elig - n_forced;
  const int kf = max(0, min(topk - n_forced, n_free));
  const float* srow = block_scores + size_t(unit) * nb_max;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = nb > 0 ? srow[min(lane + kWave * j, nb - 1)] : 0.f;
  unsigned long long chosen = 0ull, cand = 0ull;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = lane + kWave * j;
    const bool forced = i < f_init || (i >= f_loc && i < n_elig);
    if (i < n_elig) {
      if (forced) chosen |= 1ull << j; else cand |= 1ull << j;
    }
  }
  if (kf == n_free) {
    chosen |= cand;
  } else {
    for (int r = 0; r < kf; ++r) {
      float bv = -INFINITY;
      int bj = -1;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (((cand >> j) & 1ull) && (bj < 0 || v[j] > bv)) {
          bv = v[j];
          bj = j;
        }
      const float M = wave_max(bj >= 0 ? bv : -INFINITY);
      const int win = wave_min_i((bj >= 0 && bv == M) ? lane + kWave * bj : 0x7fffffff);
      if (lane == (win & (kWave - 1))) {
        const int j = win / kWave;
        chosen |= 1ull << j;
        cand &= ~(1ull << j);
      }
    }
  }
  // ascending ids: slot j then lane
  int* out = indices + size_t(unit) * topk;
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool f = (chosen >> j) & 1ull;
    const unsigned long long m = __ballot(f);
    const int pos = base + __popcll(m & below);
    if (f && pos < topk) out[pos] = lane + kWave * j;
    base += __popcll(m);
  }
  for (int i = base + lane; i < topk; i += kWave) out[i] = -1;
}

// --------------------------------------------------------------------------- host

static int n_windows_max(int max_seqlen_k) {
  return max_seqlen_k >= kKernel ? (max_seqlen_k - kKernel) / kStride + 1 : 0;
}

ScoreDims score_dims(int max_seqlen_k) {
  ScoreDims d;
  d.nc_max = n_windows_max(max_seqlen_k);
  d.nb_max = (max_seqlen_k + kBlock - 1) / kBlock;
  d.n_chunk_max = (d.nc_max + kChunkWindows - 1) / kChunkWindows;
  d.ldc = d.n_chunk_max * kChunkWindows;
  d.ldb = d.n_chunk_max * 16 + 1;
  return d;
}

static size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

size_t scores_ws_bytes(int batch, int kv_heads, int group, int max_seqlen_k) {
  const ScoreDims d = score_dims(max_seqlen_k);
  const size_t units = size_t(batch) * kv_heads;
  return up256(units * group * size_t(d.ldc) * sizeof(float)) +
         up256(units * d.n_chunk_max * group * sizeof(float2)) +
         up256(units * size_t(d.ldb) * sizeof(float));
}

ScoresWs scores_ws_carve(void* base, int batch, int kv_heads, int group, int max_seqlen_k) {
  const ScoreDims d = score_dims(max_seqlen_k);
  const size_t units = size_t(batch) * kv_heads;
  char* p = static_cast<char*>(base);
  ScoresWs ws;
  ws.logits = reinterpret_cast<float*>(p);
  p += up256(units * group * size_t(d.ldc) * sizeof(float));
  ws.part = reinterpret_cast<float2*>(p);
  p += up256(units * d.n_chunk_max * group * sizeof(float2));
  ws.cisb = reinterpret_cast<float*>(p);
  return ws;
}

template <int G, typename TQ, typename TKC>
static hipError_t launch_scores_g(const DecodeScoresArgs& a, hipStream_t s) {
  const ScoreDims d = score_dims(a.max_seqlen_k);
  float* cisb = a.cis_pooled != nullptr ? a.ws.cisb : nullptr;
  if (d.n_chunk_max > 0) {
    hipError_t e = launch_kernel(
        kKindLogits, window_logits_kernel<G, TQ, TKC>, dim3(d.n_chunk_max * a.kv_heads * a.batch),
        dim3(256), s, static_cast<const TQ*>(a.q), static_cast<TKC*>(a.kc), a.cu_k, a.cu_c,
        a.ws.logits, a.ws.part, cisb, a.cis_pooled, a.kv_heads, d.ldc, d.n_chunk_max, d.ldb,
        a.scale_log2, static_cast<const TQ*>(a.refresh_k), a.refresh_cis);
    if (e != hipSuccess) return e;
  }
  if (a.logits_only) return hipSuccess;
  return launch_kernel(kKindBlockScores, select_kernel<G, true>, dim3(a.batch * a.kv_heads),
                       dim3(kSelThreads), s, static_cast<const float*>(a.ws.logits),
                       static_cast<const float2*>(a.ws.part), static_cast<const float*>(cisb),
                       a.cis_weight, static_cast<const int*>(nullptr), a.cu_k, a.cu_c, a.batch,
                       a.block_scores, a.window_probs, a.kv_heads, d.nc_max, d.ldc, d.nb_max,
                       d.n_chunk_max, d.ldb, a.indices, a.topk, a.n_init, a.n_local, a.n_cand);
}

template <typename TQ, typename TKC>
static hipError_t launch_scores_t(int G, const DecodeScoresArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return launch_scores_g<1, TQ, TKC>(a, s);
    case 2: return launch_scores_g<2, TQ, TKC>(a, s);
    case 4: return launch_scores_g<4, TQ, TKC>(a, s);
    case 8: return launch_scores_g<8, TQ, TKC>(a, s);
    case 16: return launch_scores_g<16, TQ, TKC>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_scores(const DecodeScoresArgs& a, hipStream_t s) {
  const int G = a.heads / a.kv_heads;
  if (a.q_bf16) {
    if (a.kc_bf16) return launch_scores_t<bf16_t, bf16_t>(G, a, s);
    return launch_scores_t<bf16_t, float>(G, a, s);
  }
  if (a.kc_bf16) return launch_scores_t<float, bf16_t>(G, a, s);
  return launch_scores_t<float, float>(G, a, s);
}

template <int PER>
static hipError_t launch_select_wave(const float* block_scores, int* indices, const int* cu_q,
                                     const int* cu_k, int batch, int units, int kv_heads,
                                     int nb_max, int topk, int n_init, int n_local, hipStream_t s) {
  return launch_kernel(kKindBlockScores, select_wave_kernel<PER>, dim3((units + 3) / 4),
                       dim3(256), s, block_scores, indices, cu_q, cu_k, batch, units, kv_heads,
                       nb_max, topk, n_init, n_local);
}

hipError_t launch_select_topk(const float* block_scores, int* indices, const int* cu_q,
                              const int* cu_k, int batch, int rows_total, int kv_heads,
                              int nb_max, int topk, int n_init, int n_local, hipStream_t s) {
  if (rows_total == 0) return hipSuccess;
  if (cu_q != nullptr) {
    // prefill rows: many short rows, one wave each
    const int units = rows_total * kv_heads;
    const int per = (nb_max + kWave - 1) / kWave;
    if (per <= 1) return launch_select_wave<1>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
    if (per <= 2) return launch_select_wave<2>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
    if (per <= 4) return launch_select_wave<4>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
    if (per <= 8) return launch_select_wave<8>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
    if (per <= 16) return launch_select_wave<16>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
    if (per <= 32) return launch_select_wave<32>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
    return launch_select_wave<64>(block_scores, indices, cu_q, cu_k, batch, units, kv_heads, nb_max, topk, n_init, n_local, s);
  }
  return launch_kernel(kKindBlockScores, select_kernel<1, false>, dim3(rows_total * kv_heads),
                       dim3(kSelThreads), s, static_cast<const float*>(nullptr),
                       static_cast<const float2*>(nullptr), static_cast<const float*>(nullptr),
                       0.f, cu_q, cu_k, static_cast<const int*>(nullptr), batch,
                       const_cast<float*>(block_scores), static_cast<float*>(nullptr), kv_heads,
                       0, 0, nb_max, 0, 0, indices, topk, n_init, n_local, 0);
}

}  // namespace nsa
