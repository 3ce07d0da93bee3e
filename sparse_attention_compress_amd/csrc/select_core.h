// Block scoring from compressed-key logits and top-k block selection, as
// workgroup-level device code shared by the stand-alone selection kernel and
// the decode kernel that selects and attends in one launch.
//
// What is computed (NOSA-1B core components, component 3 stage 1; NOSA-1B source
// analysis part 3, "beyond the kernel"): for the newest token of a sequence and
// each query head h, the softmax over the visible compressed windows (its
// normaliser assembled from per-chunk (max, sum of exp2) pairs); the
// probabilities summed over the GQA group; max-pooled onto 64-token blocks
// (windows 4i-1 .. 4i+3); plus w * the pooled-CIS maximum of the block.  Then
// the selection: the first n_init and last n_local eligible blocks are forced
// in, the other places go to the best-scoring eligible blocks (ties to the lower
// id), ids ascending, -1 padded.
//
// Top-k: thread tid keeps the scores of ids tid + THREADS*u in registers; a
// histogram of order-preserving keys isolates the boundary of the k best, whose
// few candidates one wave ranks exactly; the chosen ids are written in order
// from wave ballots and one scan of the per-(slab, wave) counts.
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nsa {

template <int THREADS, int MAXB>
struct SelCfg {
  static constexpr int kThreads = THREADS;
  static constexpr int kWaves = THREADS / kWave;
  static constexpr int kPer = MAXB / THREADS;  // id slabs per thread
  static constexpr int kCounts = kPer * kWaves;
  static_assert(kCounts <= kWave, "one lane per (slab, wave) count");
  static_assert(MAXB % THREADS == 0, "whole slabs");
};

constexpr int kBins = 256;  // histogram bins of the top-k search (4 per lane of one wave)

template <int THREADS, int MAXB>
struct SelShared {
  using C = SelCfg<THREADS, MAXB>;
  int hist[2][kBins];               // alternate levels, so clearing needs no barrier
  uint32_t cand_key[kWave];         // candidates of the boundary bin (exact ranking)
  int cand_id[kWave];
  int n_cand;
  unsigned char keep[MAXB];         // chosen flags of the boundary-bin candidates
  uint32_t kred[2][C::kWaves];      // key range reduction
  int cnt[2][kWave];                // per (slab, wave) counts of the ordered scans
  float wred[2][C::kWaves][16];
  float fac[MAXB];                  // per (chunk, head): exp2(chunk max - max) / sum
  int misc[4];
};

__device__ __forceinline__ int full_windows_dev(int len) {
  return len >= kKernel ? (len - kKernel) / kStride + 1 : 0;
}

// Positions, in ascending id order, of the flagged ids; returns the number
// flagged, in every thread.  One barrier; `cnt` must not be written again
// before another barrier.
template <int THREADS, int MAXB>
__device__ __forceinline__ int ordered_positions(const bool (&flag)[SelCfg<THREADS, MAXB>::kPer],
                                                 int (&pos)[SelCfg<THREADS, MAXB>::kPer],
                                                 int* cnt) {
  using C = SelCfg<THREADS, MAXB>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < C::kPer; ++u) {
    const unsigned long long m = __ballot(flag[u]);
    pos[u] = __popcll(m & below);
    if (lane == 0) cnt[u * C::kWaves + wave] = __popcll(m);
  }
  __syncthreads();
  const int c = lane < C::kCounts ? cnt[lane] : 0;  // lane = slab * waves + wave: id order
  const int incl = wave_inclusive_scan(c);
  const int excl = incl - c;
#pragma unroll
  for (int u = 0; u < C::kPer; ++u) pos[u] += __builtin_amdgcn_readlane(excl, u * C::kWaves + wave);
  return __builtin_amdgcn_readlane(incl, kWave - 1);
}

// Selection geometry of one (row, kv head).
struct SelGeom {
  int n_elig, f_init, f_loc, n_free, kf, free_mark;
};

// With n_cand > 0 (two-stage selection) at most n_cand free blocks can be chosen.
__device__ __forceinline__ SelGeom sel_geometry(int t, int nb, int topk, int n_init, int n_local,
                                                int n_cand = 0) {
  SelGeom g;
  g.n_elig = t >= 0 ? min(nb, t / kBlock + 1) : 0;
  g.f_init = min(n_init, g.n_elig);
  g.f_loc = max(max(0, g.n_elig - n_local), g.f_init);  // forced local: [f_loc, n_elig)
  const int n_forced = g.f_init + (g.n_elig - g.f_loc);
  g.n_free = g.n_elig - n_forced;
  g.kf = max(0, min(topk - n_forced, g.n_free));
  if (n_cand > 0) g.kf = min(g.kf, n_cand);
  g.free_mark = g.kf == g.n_free ? 1 : (g.kf == 0 ? 0 : 2);
  return g;
}

// Resolves every free candidate (st == 2) to chosen (1) or dropped (0): the kf
// best by (key desc, id asc) are chosen.  Needs 0 < kf < the number of
// candidates (uniform).  A 256-bin histogram of the keys over their range (a
// shift of the key offset from the minimum, so binning is exact integer
// arithmetic) locates the bin holding the kf-th best: keys in higher bins are
// chosen, lower bins dropped.  If at most 64 candidates share that bin they are
// gathered and one wave ranks them exactly by (key desc, id asc); otherwise the
// bin is refined with the next lower bits.
template <int THREADS, int MAXB>
__device__ __forceinline__ void resolve_free(SelShared<THREADS, MAXB>& S,
                                             const uint32_t (&key)[SelCfg<THREADS, MAXB>::kPer],
                                             int (&st)[SelCfg<THREADS, MAXB>::kPer], int kf) {
  using C = SelCfg<THREADS, MAXB>;
  constexpr int P = C::kPer;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < P; ++u) {
    if (st[u] == 2) {
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
    }
  }
  // ---- key range over the workgroup
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    S.kred[0][wave] = kmin;
    S.kred[1][wave] = kmax;
  }
  for (int i = tid; i < kBins; i += THREADS) S.hist[0][i] = 0;
  if (tid == 0) S.n_cand = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) {
    kmin = min(kmin, S.kred[0][w]);
    kmax = max(kmax, S.kred[1][w]);
  }
  // offsets from kmin; the bin is the offset's top 8 significant bits
  const uint32_t span = kmax - kmin;
  int shift = span == 0u ? 0 : max(0, 24 - __clz(static_cast<int>(span)));  // span >> shift < 256
  uint32_t lo = 0u;                 // offsets of the current range: [lo, lo + (256 << shift))
  int need = kf;
  for (int level = 0; level < 5; ++level) {
    int* hist = S.hist[level & 1];
    // the other buffer was last read before the previous level's second
    // barrier and is next filled after this level's second barrier
    for (int i = tid; i < kBins; i += THREADS) S.hist[(level + 1) & 1][i] = 0;
#pragma unroll
    for (int u = 0; u < P; ++u)
      if (st[u] == 2) atomicAdd(&hist[((key[u] - kmin - lo) >> shift) & (kBins - 1)], 1);
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255-4l .. 252-4l (descending keys)
      int c[4], tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[kBins - 1 - 4 * lane - e];
        tot += c[e];
      }
      const int incl = wave_inclusive_scan(tot);
      const int above = incl - tot;
      const int r = need - above;
      int run = 0, e_star = 0, before = 0, m_star = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        run += c[e];
        const bool below = run < r;
        e_star += below ? 1 : 0;
        before += below ? c[e] : 0;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) m_star += e == e_star ? c[e] : 0;
      if (above < need && need <= incl) {
        S.misc[0] = kBins - 1 - 4 * lane - e_star;
        S.misc[1] = above + before;
        S.misc[2] = m_star;
      }
    }
    __syncthreads();
    const int bstar = S.misc[0], above = S.misc[1], m = S.misc[2];
    // decide every candidate outside the boundary bin
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (st[u] == 2) {
        const int bin = int(((key[u] - kmin - lo) >> shift) & (kBins - 1));
        if (bin != bstar) st[u] = bin > bstar ? 1 : 0;
      }
    }
    need -= above;
    if (m == need) {  // the whole bin is chosen
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (st[u] == 2) st[u] = 1;
      break;
    }
    if (m > kWave && shift == 0) {
      // more than 64 candidates share one key value: the lowest ids win
      bool f[P];
      int pos[P];
#pragma unroll
      for (int u = 0; u < P; ++u) f[u] = st[u] == 2;
      ordered_positions<THREADS, MAXB>(f, pos, S.cnt[0]);
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (f[u]) st[u] = pos[u] < need ? 1 : 0;
      break;
    }
    if (m <= kWave) {
      // gather the bin's candidates (any order: one LDS atomic per wave and
      // slab reserves their places) and rank them exactly in one wave by
      // (key desc, id asc), lane c2's candidate read back with readlane
      const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const unsigned long long bm = __ballot(st[u] == 2);
        if (bm == 0ull) continue;  // uniform in the wave
        int base = 0;
        if (lane == 0) base = atomicAdd(&S.n_cand, __popcll(bm));
        base = __builtin_amdgcn_readlane(base, 0);
        const int slot = base + __popcll(bm & below);
        if (st[u] == 2 && slot < kWave) {
          S.cand_key[slot] = key[u];
          S.cand_id[slot] = tid + THREADS * u;
        }
      }
      __syncthreads();
      if (wave == 0) {
        const int mm = min(S.n_cand, kWave);
        const uint32_t kk = lane < mm ? S.cand_key[lane] : 0u;
        const int id = lane < mm ? S.cand_id[lane] : 0x7fffffff;
        int rank = 0;
        for (int c2 = 0; c2 < mm; ++c2) {
          const uint32_t k2 = uint32_t(__builtin_amdgcn_readlane(int(kk), c2));
          const int id2 = __builtin_amdgcn_readlane(id, c2);
          rank += (k2 > kk || (k2 == kk && id2 < id)) ? 1 : 0;
        }
        if (lane < mm) S.keep[id] = rank < need ? 1 : 0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (st[u] == 2) st[u] = S.keep[tid + THREADS * u];
      break;
    }
    // refine inside the boundary bin
    lo += uint32_t(bstar) << shift;
    shift = max(0, shift - 8);
  }
}

// Top-k over the eligible ids with scores sc (registers).  Calls emit(pos, id)
// for every chosen id, pos being its place in ascending id order (pos < topk),
// and returns the number chosen (in every thread); places from that count to
// topk are the caller's to pad.  Needs no barrier before it as long as the
// caller's preceding LDS use is of other fields of S.
// One stage (n_cand <= 0): the forced ids plus the g.kf best free ids by sc.
// Two stages (n_cand > 0; g from sel_geometry with the same n_cand): the
// n_cand best free ids by sc are the candidates, and the g.kf best candidates
// by scc are chosen; ties go to the lower id in both stages.  The free scores
// become order-preserving 32-bit keys (resolve_free).  Chosen ids are then
// written in ascending order from wave ballots and one scan of the per-(slab,
// wave) counts.
template <int THREADS, int MAXB, typename Emit>
__device__ __forceinline__ int topk_select(SelShared<THREADS, MAXB>& S,
                                           const float (&sc)[SelCfg<THREADS, MAXB>::kPer],
                                           const float (&scc)[SelCfg<THREADS, MAXB>::kPer],
                                           int n_cand, const SelGeom& g, int topk, Emit&& emit) {
  using C = SelCfg<THREADS, MAXB>;
  constexpr int P = C::kPer;
  const int tid = threadIdx.x;
  int st[P];  // 0 out, 1 chosen, 2 free candidate
  uint32_t key[P];
  if (n_cand <= 0) {  // uniform
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int i = tid + THREADS * u;
      const bool forced = i < g.f_init || (i >= g.f_loc && i < g.n_elig);
      st[u] = i >= g.n_elig ? 0 : (forced ? 1 : g.free_mark);
      key[u] = float_key(sc[u] + 0.f);  // + 0 folds -0 into +0 (they compare equal)
    }
    if (g.kf > 0 && g.kf < g.n_free) resolve_free<THREADS, MAXB>(S, key, st, g.kf);  // uniform
  } else {
    bool fz[P];
    const int c1 = min(n_cand, g.n_free);  // candidates
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int i = tid + THREADS * u;
      fz[u] = i < g.f_init || (i >= g.f_loc && i < g.n_elig);
      st[u] = i >= g.n_elig ? 0 : (fz[u] ? 1 : 2);
      key[u] = float_key(sc[u] + 0.f);
    }
    if (c1 < g.n_free) resolve_free<THREADS, MAXB>(S, key, st, c1);  // c1 > 0: n_free > 0
    // stage 2 over the candidates (free ids still in)
    const int kf2 = min(g.kf, c1);
#pragma unroll
    for (int u = 0; u < P; ++u) {
      st[u] = fz[u] ? 1 : (st[u] != 0 ? (kf2 == c1 ? 1 : (kf2 == 0 ? 0 : 2)) : 0);
      key[u] = float_key(scc[u] + 0.f);
    }
    if (kf2 > 0 && kf2 < c1) {  // uniform
      __syncthreads();  // stage 1's last LDS reads are behind every thread
      resolve_free<THREADS, MAXB>(S, key, st, kf2);
    }
  }
  // ordered compaction of the chosen ids
  bool f[P];
  int pos[P];
#pragma unroll
  for (int u = 0; u < P; ++u) f[u] = st[u] == 1;
  const int total = ordered_positions<THREADS, MAXB>(f, pos, S.cnt[1]);
  // emitted places stay inside the row's topk slots even if the count were wrong
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (f[u] && pos[u] < topk) emit(pos[u], tid + THREADS * u);
  return min(total, topk);
}

// The id at place p of the ascending selection when p is not one of the free
// picks: the forced init blocks come first and the forced local blocks last
// (they are the highest eligible ids); with every eligible block chosen, place p
// holds id p.  Returns -2 for a free pick's place and -1 past the chosen count.
__device__ __forceinline__ int forced_id_at(const SelGeom& g, int p) {
  const int n_loc = g.n_elig - g.f_loc;
  const int kf = g.free_mark == 0 ? 0 : g.kf;
  if (p >= g.f_init + kf + n_loc) return -1;
  if (p < g.f_init) return p;
  if (p < g.f_init + kf) return g.free_mark == 1 ? p : -2;
  return g.f_loc + (p - g.f_init - kf);
}

// (max, sum of exp2) of the union of two sets of log2-domain logits.
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  l = (m == -INFINITY ? 0.f : l * fast_exp2(m - M)) + (m2 == -INFINITY ? 0.f : l2 * fast_exp2(m2 - M));
  m = M;
}

// ml_merge over the lanes that share lane % G (G a power of two <= 16): rotations
// by 2, 4, 8 inside a row (for G = 1 the four quad / mirror steps), then the two
// row-pair swaps; the result for column lane % G lands in all of them.
template <int G>
__device__ __forceinline__ void column_merge_ml(float& m, float& l) {
  auto dpp_step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    ml_merge(m, l, dpp<C>(m), dpp<C>(l));
  };
  if constexpr (G == 1) {
    dpp_step(std::integral_constant<int, kDppQuadXor1>());
    dpp_step(std::integral_constant<int, kDppQuadXor2>());
    dpp_step(std::integral_constant<int, kDppRowHalfMirror>());
    dpp_step(std::integral_constant<int, kDppRowMirror>());
  } else {
    if constexpr (G <= 2) dpp_step(std::integral_constant<int, kDppRowRor2>());
    if constexpr (G <= 4) dpp_step(std::integral_constant<int, kDppRowRor4>());
    if constexpr (G <= 8) dpp_step(std::integral_constant<int, kDppRowRor8>());
  }
  // rows pair up through the two lane swaps (both results are {own, partner})
  {
    auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    auto rl = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    m = __uint_as_float(rm[0]);
    l = __uint_as_float(rl[0]);
    ml_merge(m, l, __uint_as_float(rm[1]), __uint_as_float(rl[1]));
  }
  {
    auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    m = __uint_as_float(rm[0]);
    l = __uint_as_float(rl[0]);
    ml_merge(m, l, __uint_as_float(rm[1]), __uint_as_float(rl[1]));
  }
}

// Inputs of block_scores_from_logits held in registers: the chunk (max, sum)
// pairs, the windows 4i-1 .. 4i+3 of every head for the first kPre id slabs
// (later slabs are loaded after the normaliser), and the block CIS maxima.
template <int G, int THREADS, int MAXB>
struct ScoreInputs {
  static constexpr int kPer = SelCfg<THREADS, MAXB>::kPer;
  static constexpr int kPairs = (MAXB + THREADS - 1) / THREADS;  // n_chunk * G <= MAXB pairs
  static constexpr int kPre = kPer < 2 ? kPer : (G > 8 ? 1 : 2);
  float2 ml[kPairs];
  float4 lg4[kPre][G];
  float lgp[kPre][G];
  float cv[kPer];
};

// Window logits of id slab u (blocks tid + THREADS*u) of one unit's rows: the
// float4 of windows 4i .. 4i+3 and window 4i-1 for every head, the column
// clamped into the row (ldc is a multiple of 64 and at least 64).
template <int G, int THREADS>
__device__ __forceinline__ void load_window_slab(const float* __restrict__ lrow, int ldc, int u,
                                                 float4 (&w4)[G], float (&wp)[G]) {
  const int c0 = min(4 * (int(threadIdx.x) + THREADS * u), ldc - 4);
  const int cp = max(c0 - 1, 0);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    w4[h] = *reinterpret_cast<const float4*>(lrow + size_t(h) * ldc + c0);
    wp[h] = lrow[size_t(h) * ldc + cp];
  }
}

// Issues the loads of ScoreInputs.  Their addresses depend only on the unit and
// the buffer geometry (n_chunk_max, ldc, ldb), not on the sequence's length, so
// a kernel calls this first and the loads overlap its wait for the sequence
// offsets; every index is clamped into the unit's rows and block_scores_from_logits
// ignores the values past the sequence's windows and blocks.  With no window
// buffer at all (n_chunk_max == 0) nothing is loaded.
template <int G, int THREADS, int MAXB>
__device__ __forceinline__ void load_score_inputs(ScoreInputs<G, THREADS, MAXB>& in,
                                                  const float* __restrict__ logits,
                                                  const float2* __restrict__ part,
                                                  const float* __restrict__ cisb, size_t unit,
                                                  int n_chunk_max, int ldc, int ldb) {
  using In = ScoreInputs<G, THREADS, MAXB>;
  const int tid = threadIdx.x;
  const bool any = n_chunk_max > 0;  // uniform
  const float2* prow = part + unit * n_chunk_max * G;
#pragma unroll
  for (int u = 0; u < In::kPairs; ++u)
    in.ml[u] = any ? prow[min(tid + THREADS * u, n_chunk_max * G - 1)] : make_float2(-INFINITY, 0.f);
  const float* lrow = logits + unit * G * ldc;
#pragma unroll
  for (int u = 0; u < In::kPre; ++u) {
    if (any) {
      load_window_slab<G, THREADS>(lrow, ldc, u, in.lg4[u], in.lgp[u]);
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        in.lg4[u][h] = make_float4(0.f, 0.f, 0.f, 0.f);
        in.lgp[u][h] = 0.f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < In::kPer; ++u)
    in.cv[u] = cisb != nullptr ? cisb[unit * ldb + min(tid + THREADS * u, ldb - 1)] : 0.f;
}

// Block scores of one decode (sequence, kv head) from the compressed-key logits
// kernel's outputs (per window and head e = exp2(logit - chunk max) [unit][G][ldc],
// chunk (max, sum) pairs [unit][n_chunk_max][G], block CIS maxima [unit][ldb]),
// given the inputs load_score_inputs fetched for the same unit:
// sc[u] for block i = tid + THREADS*u (u < slabs holding ids < nb; 0 elsewhere).
// P_h(c) = e_h(c) * exp2(m_h(chunk) - M_h) / L_h, the per-(chunk, head) factor
// computed once per workgroup into LDS.  The thread owning block i reads the
// values of its windows 4i-1 .. 4i+3 itself, so no window value crosses threads.
// With split_cis (two-stage selection) sc holds the attention part alone and
// scc the block CIS maxima; otherwise sc = attention part + cis_weight * CIS
// maximum and scc is 0.  Optional debug outputs: block_scores [unit][nb_max]
// (sc; 0 past nb) and window_probs [unit][nc_max].  Two workgroup barriers.
template <int G, int THREADS, int MAXB>
__device__ __forceinline__ void block_scores_from_logits(
    SelShared<THREADS, MAXB>& S, float (&sc)[SelCfg<THREADS, MAXB>::kPer],
    float (&scc)[SelCfg<THREADS, MAXB>::kPer], bool split_cis,
    ScoreInputs<G, THREADS, MAXB>& in, const float* __restrict__ logits,
    const float* __restrict__ cisb, float cis_weight, size_t unit, int nvis, int nb,
    int ldc, int nb_max, int nc_max, float* __restrict__ block_scores,
    float* __restrict__ window_probs) {
  using C = SelCfg<THREADS, MAXB>;
  using In = ScoreInputs<G, THREADS, MAXB>;
  constexpr int P = C::kPer;
  constexpr int kPairs = In::kPairs;
  constexpr int kPre = In::kPre;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_slab = (nb + THREADS - 1) / THREADS;  // uniform
  const int n_chunk = (nvis + kChunkWindows - 1) / kChunkWindows;
  const int n_pairs = n_chunk * G;
  const float* lrow = logits + unit * G * ldc;
  const bool with_cis = cisb != nullptr && n_chunk > 0;

  // per-head softmax normaliser: merge of the chunk pairs; pair i of this
  // thread belongs to head i % G == tid % G
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int u = 0; u < kPairs; ++u)
    if (tid + THREADS * u < n_pairs) ml_merge(m, l, in.ml[u].x, in.ml[u].y);
  column_merge_ml<G>(m, l);
  if (lane < G) {
    S.wred[0][wave][lane] = m;
    S.wred[1][wave][lane] = l;
  }
  __syncthreads();
  {
    const int h = tid % G;
    float Mh = -INFINITY, Lh = 0.f;
#pragma unroll
    for (int w = 0; w < C::kWaves; ++w) ml_merge(Mh, Lh, S.wred[0][w][h], S.wred[1][w][h]);
    const float invL = 1.f / Lh;
    // factor of each (chunk, head) pair this thread loaded
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int p = tid + THREADS * u;
      if (p < n_pairs) S.fac[p] = in.ml[u].x == -INFINITY ? 0.f : fast_exp2(in.ml[u].x - Mh) * invL;
    }
  }
  __syncthreads();
  // group probabilities of the block's windows 4i-1 .. 4i+3, their max, + CIS
  const int owned = with_cis ? min(nb, 16 * n_chunk + 1) : 0;
  auto score_slab = [&](int u, const float4 (&w4)[G], const float (&wp)[G]) {
    const int i = tid + THREADS * u;
    // windows 4i .. 4i+3 lie in chunk i/16; window 4i-1 in chunk (4i-1)/64
    const int j0 = min(i / 16, max(n_chunk - 1, 0));
    const int jp = min(max(4 * i - 1, 0) / kChunkWindows, max(n_chunk - 1, 0));
    float pg[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float f0 = S.fac[j0 * G + h], fp = S.fac[jp * G + h];
      pg[0] += wp[h] * fp;
      pg[1] += w4[h].x * f0;
      pg[2] += w4[h].y * f0;
      pg[3] += w4[h].z * f0;
      pg[4] += w4[h].w * f0;
    }
    float pm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 5; ++e) {
      const int c = 4 * i - 1 + e;
      if (c >= 0 && c < nvis) pm = fmaxf(pm, pg[e]);
    }
    float s = pm == -INFINITY ? 0.f : pm;
    if (cisb != nullptr) {
      const float cv = i < owned ? in.cv[u] : 0.f;
      if (split_cis)
        scc[u] = cv;
      else
        s += cis_weight * cv;
    }
    if (block_scores != nullptr && i < nb) block_scores[unit * nb_max + i] = s;
    if (window_probs != nullptr) {
#pragma unroll
      for (int e = 1; e < 5; ++e) {
        const int c = 4 * i - 1 + e;
        if (c < nc_max) window_probs[unit * nc_max + c] = c < nvis ? pg[e] : 0.f;
      }
    }
    return s;
  };
  // Slab u is scored from preload set u % kPre, which then takes the loads of
  // slab u + kPre: kPre slabs stay in flight.  Those loads are issued whether or
  // not the slab holds blocks of this row (addresses clamped into the unit's
  // rows), so no branch makes the wait counts conservative.
#pragma unroll
  for (int u = 0; u < P; ++u) {
    sc[u] = 0.f;
    scc[u] = 0.f;
    constexpr int kSets = kPre > 0 ? kPre : 1;
    if (u < n_slab) sc[u] = score_slab(u, in.lg4[u % kSets], in.lgp[u % kSets]);
    if (u + kPre < P && ldc > 0)
      load_window_slab<G, THREADS>(lrow, ldc, u + kPre, in.lg4[u % kSets], in.lgp[u % kSets]);
  }
  if (block_scores != nullptr)
    for (int i = nb + tid; i < nb_max; i += THREADS) block_scores[unit * nb_max + i] = 0.f;
  if (window_probs != nullptr)
    for (int c = 4 * nb + tid; c < nc_max; c += THREADS) window_probs[unit * nc_max + c] = 0.f;
}

}  // namespace nsa
