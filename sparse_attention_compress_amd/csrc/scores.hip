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
// window_logits_kernel -- grid (chunk of 64 windows, kv head, sequence).  Each
//   wave scores 16 windows; a quad of lanes shares one compressed-key row (each
//   lane a 32-dim slice, 16-byte loads) and the G query heads of the group come
//   from LDS, so each compressed key is read from HBM once for the whole group.
//   It writes log2-domain logits and a per-chunk (max, sum of exp2) per head.
//   Optionally the workgroup owning the newest window first recomputes that
//   window of the K_c and pooled-CIS caches from K and CIS (decode refresh).
// select_kernel -- one workgroup of 1024 threads per (row, kv head).  Either
//   derives the block scores from the logits (decode) or reads given scores,
//   then selects: forced blocks, and among the others a histogram of the scores
//   over [min, max] locates the bin holding the k-th best, blocks above it are
//   taken and the bin's candidates are ranked exactly by (score desc, id asc);
//   chosen ids are written in ascending order by a workgroup scan.
// No kernel waits on another workgroup: every hand-off is a kernel boundary.
#include "common.h"
#include "launch.h"

namespace nsa {

__device__ __forceinline__ int full_windows_dev(int len) {
  return len >= kKernel ? (len - kKernel) / kStride + 1 : 0;
}

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

template <int G, typename TQ, typename TKC>
__global__ __launch_bounds__(256) void window_logits_kernel(
    const TQ* __restrict__ q, TKC* __restrict__ kc, const int* __restrict__ cu_k,
    const int* __restrict__ cu_c, float* __restrict__ logits, float2* __restrict__ part,
    int kv_heads, int nc_max, int n_chunk_max, float scale_log2,
    const TQ* __restrict__ k_src, const float* __restrict__ cis_src, float* __restrict__ cis_pooled) {
  __shared__ float q_s[G][kHeadDim];
  __shared__ float new_s[kHeadDim];
  __shared__ float red_s[4][G];
  __shared__ float m_s[G];
  const int b = blockIdx.z, kv = blockIdx.y, chunk = blockIdx.x;
  const int start = cu_k[b];
  const int len = cu_k[b + 1] - start;
  const int cbase = cu_c[b];
  const int nc = cu_c[b + 1] - cbase;
  const int nvis = min(nc, full_windows_dev(len));  // decode query at t = len-1
  const int c0 = chunk * kChunkWindows;
  if (c0 >= nvis) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c = c0 + wave * 16 + (lane >> 2);
  const int r = lane & 3;
  const bool valid = c < nvis;
  // window refreshed from K in this workgroup (decode append), else -1
  const int rw = (k_src != nullptr && nvis == nc && nc - 1 >= c0 && nc - 1 < c0 + kChunkWindows)
                     ? nc - 1 : -1;

  // issue every global load of the workgroup before the first use
  float kf[4][8];
  if (valid && c != rw) {
    const TKC* row = kc + (size_t(cbase + c) * kv_heads + kv) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) load8f(row + 32 * i + 8 * r, kf[i]);
  }
  float racc = 0.f, rcis = 0.f;
  if (rw >= 0) {
    const int j0 = start + kStride * rw;
    if (tid < kHeadDim) {
      // same summation order as the pooling kernel: token by token
      float xv[kKernel];
#pragma unroll
      for (int j = 0; j < kKernel; ++j)
        xv[j] = to_f32(k_src[(size_t(j0 + j) * kv_heads + kv) * kHeadDim + tid]);
#pragma unroll
      for (int j = 0; j < kKernel; ++j) racc += xv[j];
      racc = racc / float(kKernel);
    } else if (cis_src != nullptr && tid >= 128 && tid < 128 + kKernel) {
      rcis = cis_src[size_t(j0 + tid - 128) * kv_heads + kv];
    }
  }
  const TQ* qg = q + (size_t(b) * kv_heads + kv) * G * kHeadDim;
  for (int i = tid; i < G * kHeadDim; i += 256) q_s[i / kHeadDim][i % kHeadDim] = to_f32(qg[i]);
  if (rw >= 0) {
    if (tid < kHeadDim) {
      new_s[tid] = racc;
      store_f32(kc + (size_t(cbase + rw) * kv_heads + kv) * kHeadDim + tid, racc);
    }
    if (cis_src != nullptr && cis_pooled != nullptr && wave == 2) {
      // lanes 0..31 of wave 2 hold the window's 32 scores, in token order
      float x = lane < kKernel ? rcis : 0.f;
      float acc = 0.f;
      for (int j = 0; j < kKernel; ++j) acc += __shfl(x, j, kWave);
      if (lane == 0) cis_pooled[size_t(cbase + rw) * kv_heads + kv] = acc / float(kKernel);
    }
  }
  __syncthreads();
  if (valid && c == rw) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = new_s[32 * i + 8 * r + e];
      // what a reader of the cache sees: the value rounded to the cache dtype
      TKC st[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) store_f32(&st[e], tmp[e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[i][e] = to_f32(st[e]);
    }
  }
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  if (valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float* qq = &q_s[h][32 * i + 8 * r];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[h] = fmaf(qq[e], kf[i][e], s[h]);
      }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s[h] += __shfl_xor(s[h], 1, kWave);
    s[h] += __shfl_xor(s[h], 2, kWave);
    s[h] = valid ? s[h] * scale_log2 : -INFINITY;
  }
  const size_t unit = size_t(b) * kv_heads + kv;
  if (valid) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      if ((h & 3) == r) logits[(unit * G + h) * nc_max + c] = s[h];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = wave_max(s[h]);
    if (lane == 0) red_s[wave][h] = m;
  }
  __syncthreads();
  if (tid < G) m_s[tid] = fmaxf(fmaxf(red_s[0][tid], red_s[1][tid]), fmaxf(red_s[2][tid], red_s[3][tid]));
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p = (valid && r == 0) ? fast_exp2(s[h] - m_s[h]) : 0.f;
    const float l = wave_sum(p);
    if (lane == 0) red_s[wave][h] = l;
  }
  __syncthreads();
  if (tid < G)
    part[(unit * n_chunk_max + chunk) * G + tid] =
        make_float2(m_s[tid], red_s[0][tid] + red_s[1][tid] + red_s[2][tid] + red_s[3][tid]);
}

// ------------------------------------------------------------ kernel 2: select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 1024;

struct SelShared {
  float sc[kMaxSortBlocks];                 // block scores of the row
  unsigned long long cand[kMaxSortBlocks];  // candidate keys (score key, ~id)
  int hist[kBins];
  unsigned char sel[kMaxSortBlocks];
  float wred[2][kSelWaves];
  int wsum[kSelWaves + 1];
  int misc[4];
  float fmisc[4];
};

__device__ __forceinline__ float block_reduce_max(float x, SelShared& S, int slot) {
  x = wave_max(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) S.wred[slot][wave] = x;
  __syncthreads();
  float m = S.wred[slot][0];
  for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, S.wred[slot][w]);
  return m;
}

// exclusive scan of per-thread counts over the workgroup; returns the thread's
// offset, total in S.wsum[kSelWaves]
__device__ __forceinline__ int block_exclusive_scan(int cnt, SelShared& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) S.wsum[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const int v = S.wsum[w];
      S.wsum[w] = run;
      run += v;
    }
    S.wsum[kSelWaves] = run;
  }
  __syncthreads();
  return S.wsum[wave] + incl - cnt;
}

// Top-k of S.sc[0..nb) for query position t; writes topk ids to out.
__device__ void topk_select(SelShared& S, int nb, int t, int topk, int n_init, int n_local,
                            int* __restrict__ out) {
  const int tid = threadIdx.x;
  const int n_elig = t >= 0 ? min(nb, t / kBlock + 1) : 0;
  const int f_init = min(n_init, n_elig);
  const int f_loc = max(max(0, n_elig - n_local), f_init);  // forced local: [f_loc, n_elig)
  const int n_forced = f_init + (n_elig - f_loc);
  const int n_free = n_elig - n_forced;
  const int kf = max(0, min(topk - n_forced, n_free));
  for (int i = tid; i < n_elig; i += kSelThreads)
    S.sel[i] = (i < f_init || i >= f_loc || kf == n_free) ? 1 : 0;
  if (kf > 0 && kf < n_free) {
    // range of the free scores
    float lo = INFINITY, hi = -INFINITY;
    for (int i = f_init + tid; i < f_loc; i += kSelThreads) {
      lo = fminf(lo, S.sc[i]);
      hi = fmaxf(hi, S.sc[i]);
    }
    const float vmax = block_reduce_max(hi, S, 0);
    const float vmin = -block_reduce_max(-lo, S, 1);
    const float width = vmax - vmin;
    const float scale = float(kBins) / width;
    const bool binned = width > 0.f && isfinite(scale) && isfinite(width);
    int above = 0, bstar = 0;
    if (binned) {
      for (int i = tid; i < kBins; i += kSelThreads) S.hist[i] = 0;
      __syncthreads();
      for (int i = f_init + tid; i < f_loc; i += kSelThreads) {
        const int bin = min(kBins - 1, int((S.sc[i] - vmin) * scale));
        atomicAdd(&S.hist[bin], 1);
      }
      __syncthreads();
      // suffix counts from the top bin: thread j owns bin kBins-1-j
      const int j = tid;
      const int cnt = j < kBins ? S.hist[kBins - 1 - j] : 0;
      const int excl = block_exclusive_scan(cnt, S);  // blocks in higher bins
      if (j < kBins && excl < kf && kf <= excl + cnt) {
        S.misc[0] = kBins - 1 - j;
        S.misc[1] = excl;
      }
      __syncthreads();
      bstar = S.misc[0];
      above = S.misc[1];
    }
    // candidates: the bin holding the k-th best (every free block when unbinned)
    if (tid == 0) S.misc[2] = 0;
    __syncthreads();
    for (int i = f_init + tid; i < f_loc; i += kSelThreads) {
      const float v = S.sc[i];
      const int bin = binned ? min(kBins - 1, int((v - vmin) * scale)) : 0;
      if (bin > bstar) {
        S.sel[i] = 1;
      } else if (bin == bstar) {
        const int pos = atomicAdd(&S.misc[2], 1);
        S.cand[pos] = (static_cast<unsigned long long>(float_key(v)) << 32) |
                      static_cast<unsigned long long>(0xffffffffu - unsigned(i));
      }
    }
    __syncthreads();
    const int m = S.misc[2];
    const int need = kf - above;
    if (m <= kSelThreads) {
      // exact rank among the candidates (keys are distinct)
      if (tid < m) {
        const unsigned long long mine = S.cand[tid];
        int rank = 0;
        for (int o = 0; o < m; ++o) rank += S.cand[o] > mine ? 1 : 0;
        if (rank < need) S.sel[0xffffffffu - unsigned(mine & 0xffffffffull)] = 1;
      }
    } else {
      // many candidates: bitonic sort of their keys, descending
      int n = 64;
      while (n < m) n <<= 1;
      for (int i = m + tid; i < n; i += kSelThreads) S.cand[i] = 0ull;
      __syncthreads();
      for (int k2 = 2; k2 <= n; k2 <<= 1) {
        for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
          for (int i = tid; i < (n >> 1); i += kSelThreads) {
            const int a_i = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
            const int b_i = a_i | jj;
            const unsigned long long a = S.cand[a_i], c = S.cand[b_i];
            if ((a < c) == ((a_i & k2) == 0)) {
              S.cand[a_i] = c;
              S.cand[b_i] = a;
            }
          }
          __syncthreads();
        }
      }
      for (int i = tid; i < need; i += kSelThreads)
        S.sel[0xffffffffu - unsigned(S.cand[i] & 0xffffffffull)] = 1;
    }
  }
  __syncthreads();
  // ordered compaction: thread tid owns ids [tid*per, tid*per+per)
  const int per = (n_elig + kSelThreads - 1) / kSelThreads;
  const int i0 = tid * per;
  int cnt = 0;
  for (int i = i0; i < min(i0 + per, n_elig); ++i) cnt += S.sel[i];
  int pos = block_exclusive_scan(cnt, S);
  for (int i = i0; i < min(i0 + per, n_elig); ++i)
    if (S.sel[i]) out[pos++] = i;
  const int total = S.wsum[kSelWaves];
  for (int i = total + tid; i < topk; i += kSelThreads) out[i] = -1;
}

template <int G, bool FROM_LOGITS>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ logits, const float2* __restrict__ part,
    const float* __restrict__ cis_pooled, float cis_weight, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, const int* __restrict__ cu_c, int batch,
    float* __restrict__ block_scores, float* __restrict__ window_probs, int kv_heads,
    int nc_max, int nb_max, int n_chunk_max, int* __restrict__ indices, int topk, int n_init,
    int n_local) {
  __shared__ SelShared S;
  __shared__ float hm_s[kSelWaves][G], hl_s[kSelWaves][G];
  __shared__ float M_s[G], invL_s[G];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x, kv = blockIdx.y;
  int b, t;
  row_position(row, cu_q, cu_k, batch, b, t);
  const int len = cu_k[b + 1] - cu_k[b];
  const int nb = min(nb_max, (len + kBlock - 1) / kBlock);
  const size_t unit = size_t(row) * kv_heads + kv;

  if constexpr (FROM_LOGITS) {
    const int cbase = cu_c[b];
    const int nc = cu_c[b + 1] - cbase;
    const int nvis = min(nc, full_windows_dev(len));
    const int n_chunk = (nvis + kChunkWindows - 1) / kChunkWindows;
    // per-head softmax normaliser from the chunk (max, sum) pairs
    constexpr int kPer = 4;  // chunk pairs per thread (n_chunk * G <= 4096)
    float2 ml[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      ml[u] = i < n_chunk * G ? part[(unit * n_chunk_max + i / G) * G + i % G]
                              : make_float2(-INFINITY, 0.f);
    }
    // thread tid always sees head tid % G (kSelThreads is a multiple of G)
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPer; ++u) m = fmaxf(m, ml[u].x);
#pragma unroll
    for (int o = G; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if (lane < G) hm_s[wave][lane] = m;
    __syncthreads();
    if (tid < G) {
      float mm = hm_s[0][tid];
      for (int w = 1; w < kSelWaves; ++w) mm = fmaxf(mm, hm_s[w][tid]);
      M_s[tid] = mm;
    }
    __syncthreads();
    const float Mh = M_s[tid % G];
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (ml[u].x != -INFINITY) l += ml[u].y * fast_exp2(ml[u].x - Mh);
#pragma unroll
    for (int o = G; o < kWave; o <<= 1) l += __shfl_xor(l, o, kWave);
    if (lane < G) hl_s[wave][lane] = l;
    __syncthreads();
    if (tid < G) {
      float ll = 0.f;
      for (int w = 0; w < kSelWaves; ++w) ll += hl_s[w][tid];
      invL_s[tid] = 1.f / ll;
    }
    __syncthreads();
    // block scores: windows 4i-1 .. 4i+3 overlap block i
    for (int i = tid; i < nb; i += kSelThreads) {
      float lg[5][G];
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const int c = 4 * i - 1 + e;
#pragma unroll
        for (int h = 0; h < G; ++h)
          lg[e][h] = (c >= 0 && c < nvis) ? logits[(unit * G + h) * nc_max + c] : -INFINITY;
      }
      float cw[5];
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const int c = 4 * i - 1 + e;
        cw[e] = (cis_pooled != nullptr && c >= 0 && c < nc)
                    ? cis_pooled[(size_t(cbase) + c) * kv_heads + kv] : -INFINITY;
      }
      float pm = -INFINITY, cm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const int c = 4 * i - 1 + e;
        if (c >= 0 && c < nvis) {
          float pg = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) pg += fast_exp2(lg[e][h] - M_s[h]) * invL_s[h];
          pm = fmaxf(pm, pg);
        }
        cm = fmaxf(cm, cw[e]);
      }
      float sc = pm == -INFINITY ? 0.f : pm;
      if (cis_pooled != nullptr) sc += cis_weight * (cm == -INFINITY ? 0.f : cm);
      S.sc[i] = sc;
      if (block_scores != nullptr) block_scores[unit * nb_max + i] = sc;
    }
    if (block_scores != nullptr)
      for (int i = nb + tid; i < nb_max; i += kSelThreads) block_scores[unit * nb_max + i] = 0.f;
    if (window_probs != nullptr) {
      for (int c = tid; c < nc_max; c += kSelThreads) {
        float pg = 0.f;
        if (c < nvis) {
#pragma unroll
          for (int h = 0; h < G; ++h)
            pg += fast_exp2(logits[(unit * G + h) * nc_max + c] - M_s[h]) * invL_s[h];
        }
        window_probs[unit * nc_max + c] = pg;
      }
    }
  } else {
    for (int i = tid; i < nb; i += kSelThreads) S.sc[i] = block_scores[unit * nb_max + i];
  }
  if (indices == nullptr) return;
  __syncthreads();
  topk_select(S, nb, t, topk, n_init, n_local, indices + unit * topk);
}

// --------------------------------------------------------------------------- host

static int n_windows_max(int max_seqlen_k) {
  return max_seqlen_k >= kKernel ? (max_seqlen_k - kKernel) / kStride + 1 : 0;
}

size_t scores_ws_bytes(int batch, int kv_heads, int group, int nc_max) {
  const size_t units = size_t(batch) * kv_heads;
  const size_t n_chunk = (size_t(nc_max) + kChunkWindows - 1) / kChunkWindows;
  size_t bytes = (units * group * size_t(nc_max) * sizeof(float) + 255) & ~size_t(255);
  bytes += (units * n_chunk * group * sizeof(float2) + 255) & ~size_t(255);
  return bytes;
}

ScoresWs scores_ws_carve(void* base, int batch, int kv_heads, int group, int nc_max) {
  const size_t units = size_t(batch) * kv_heads;
  char* p = static_cast<char*>(base);
  ScoresWs ws;
  ws.logits = reinterpret_cast<float*>(p);
  p += (units * group * size_t(nc_max) * sizeof(float) + 255) & ~size_t(255);
  ws.part = reinterpret_cast<float2*>(p);
  return ws;
}

template <int G, typename TQ, typename TKC>
static hipError_t launch_scores_g(const DecodeScoresArgs& a, hipStream_t s) {
  const int nc_max = n_windows_max(a.max_seqlen_k);
  const int nb_max = (a.max_seqlen_k + kBlock - 1) / kBlock;
  const int n_chunk_max = (nc_max + kChunkWindows - 1) / kChunkWindows;
  if (n_chunk_max > 0) {
    hipError_t e = launch_kernel(
        kKindLogits, window_logits_kernel<G, TQ, TKC>, dim3(n_chunk_max, a.kv_heads, a.batch),
        dim3(256), s, static_cast<const TQ*>(a.q), static_cast<TKC*>(a.kc), a.cu_k, a.cu_c,
        a.ws.logits, a.ws.part, a.kv_heads, nc_max, n_chunk_max, a.scale_log2,
        static_cast<const TQ*>(a.refresh_k), a.refresh_cis, a.refresh_cis_pooled);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(kKindBlockScores, select_kernel<G, true>, dim3(a.batch, a.kv_heads),
                       dim3(kSelThreads), s, static_cast<const float*>(a.ws.logits),
                       static_cast<const float2*>(a.ws.part), a.cis_pooled, a.cis_weight,
                       static_cast<const int*>(nullptr), a.cu_k, a.cu_c, a.batch, a.block_scores,
                       a.window_probs, a.kv_heads, nc_max, nb_max, n_chunk_max, a.indices, a.topk,
                       a.n_init, a.n_local);
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

hipError_t launch_select_topk(const float* block_scores, int* indices, const int* cu_q,
                              const int* cu_k, int batch, int rows_total, int kv_heads,
                              int nb_max, int topk, int n_init, int n_local, hipStream_t s) {
  if (rows_total == 0) return hipSuccess;
  return launch_kernel(kKindBlockScores, select_kernel<1, false>, dim3(rows_total, kv_heads),
                       dim3(kSelThreads), s, static_cast<const float*>(nullptr),
                       static_cast<const float2*>(nullptr), static_cast<const float*>(nullptr),
                       0.f, cu_q, cu_k, static_cast<const int*>(nullptr), batch,
                       const_cast<float*>(block_scores), static_cast<float*>(nullptr), kv_heads,
                       0, nb_max, 0, indices, topk, n_init, n_local);
}

}  // namespace nsa
