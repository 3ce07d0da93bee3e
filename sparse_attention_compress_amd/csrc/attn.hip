// Attention over selected KV blocks, GQA-grouped.
//
// What is computed (NOSA-1B core components, decode stage; TileLang NSA,
// section 2): for a query row at position t and KV head g, the G query heads of
// group g attend to every token j <= t of every listed block id (ids < 0 or with
// 64*id > t are skipped), softmax(scale * q.k) . v; in CIS mode the softmax
// weights are multiplied by cis_j and renormalised (values scaled by CIS,
// divided by the same attention over all-ones values).
//
// Design (gfx950; decode is HBM-bound): one workgroup of 4 waves serves one
// (row, kv head) and a run of selected blocks.  Wave w owns tokens 16w..16w+15
// of every block and keeps its own online-softmax state, so the block loop has
// no workgroup barrier.  The K/V of the next block are loaded into a second
// register buffer while the current block is computed, and every selected K/V
// byte is fetched from HBM once for the whole query group.  Softmax runs in the
// exp2 domain (log2 e folded into the scale).  Two variants:
//   * bf16 (decode and prefill rows): both products on the matrix cores (see
//     selected_attn_mfma_kernel);
//   * float32 (the fp32 decode configuration): on the vector ALUs; for q.k a
//     quad of lanes shares a key row (each lane a 32-dim slice via 16-byte
//     loads, the G query heads from LDS); for p.v each lane owns 8 dims of 4
//     tokens, so V rows are read as whole 256-byte lines.
// Decode splits the selected blocks of a (row, kv head) over several workgroups
// that write partial (max, sum, acc); combine_kernel merges them.  The decode
// step runs the selection inside that kernel (select_attn_kernel).  Prefill
// rows use one workgroup per (row, kv head) and write the output directly.
#include "common.h"
#include "launch.h"
#include "select_core.h"

namespace nsa {

template <typename T>
struct Row8;

template <>
struct Row8<bf16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = ld16(p); }
  __device__ __forceinline__ void zero() { r = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ float f(int e) const {
    const uint32_t x = (e >> 1) == 0 ? r.x : (e >> 1) == 1 ? r.y : (e >> 1) == 2 ? r.z : r.w;
    return (e & 1) ? bf16hi(x) : bf16lo(x);
  }
};

template <>
struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0.f, 0.f, 0.f, 0.f);
    b = a;
  }
  __device__ __forceinline__ float f(int e) const {
    switch (e) {
      case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
      case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
    }
  }
};

template <typename T>
struct BlockRegs {
  Row8<T> k[4];  // q.k slice of this lane's token
  Row8<T> v[4];  // p.v slice of this lane's 4 tokens
  float cw;      // CIS weight of this lane's q.k token
};

__device__ __forceinline__ void attn_row_position(int row, const int* __restrict__ cu_q,
                                                  const int* __restrict__ cu_k, int batch,
                                                  int& b, int& t) {
  if (cu_q == nullptr) {
    b = row;
    t = cu_k[b + 1] - cu_k[b] - 1;
    return;
  }
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  b = lo;
  t = (row - cu_q[b]) + ((cu_k[b + 1] - cu_k[b]) - (cu_q[b + 1] - cu_q[b]));
}

constexpr int kMaxWgSlots = 64;  // selected-block slots one workgroup stages at once

template <int G, typename T, bool CIS, bool SPLIT>
__global__ __launch_bounds__(256) void selected_attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int* __restrict__ indices, int k_sel, const float* __restrict__ cis,
    T* __restrict__ out, float* __restrict__ lse, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int batch, int kv_heads, float scale_log2, int bpw,
    float2* __restrict__ part_ml, float* __restrict__ part_acc) {
  constexpr int D = kHeadDim;
  constexpr bool kBF16 = sizeof(T) == 2;
  __shared__ uint32_t q_s[kBF16 ? G * D / 2 : G * D];  // bf16 pairs or fp32 values
  __shared__ float p_s[4][16][G];
  __shared__ float m_s[4][G], l_s[4][G];
  __shared__ float acc_s[4][G][D];
  __shared__ int ids_s[kMaxWgSlots];
  __shared__ int nv_s;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kv = blockIdx.y;
  const int row = SPLIT ? int(blockIdx.z) : int(blockIdx.x);
  const int split = SPLIT ? int(blockIdx.x) : 0;
  int b, t;
  attn_row_position(row, cu_q, cu_k, batch, b, t);
  const int kstart = cu_k[b];
  const size_t unit = size_t(row) * kv_heads + kv;
  const int s_begin = split * bpw;
  const int s_end = SPLIT ? min(k_sel, s_begin + bpw) : k_sel;

  // stage the usable block ids of this workgroup (in list order) and the queries
  if (wave == 0) {
    int base = 0;
    for (int s0 = s_begin; s0 < s_end; s0 += kWave) {
      const int sl = s0 + lane;
      const int id = sl < s_end ? indices[unit * k_sel + sl] : -1;
      const bool ok = id >= 0 && id * kBlock <= t;
      const unsigned long long mask = __ballot(ok);
      const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
      if (ok && pos < kMaxWgSlots) ids_s[pos] = id;
      base += __popcll(mask);
    }
    if (lane == 0) nv_s = min(base, kMaxWgSlots);
  }
  {
    const uint32_t* qg = reinterpret_cast<const uint32_t*>(q + unit * G * D);
    constexpr int kWords = kBF16 ? G * D / 2 : G * D;
#pragma unroll
    for (int i = 0; i < (kWords + 255) / 256; ++i)
      if (tid + 256 * i < kWords) q_s[tid + 256 * i] = qg[tid + 256 * i];
  }
  __syncthreads();
  const int nv = nv_s;

  const int tok = lane >> 2, r = lane & 3;   // q.k: token of the wave, 32-dim slice
  const int u = lane >> 4, o = lane & 15;    // p.v: token quarter, 8-dim slice
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }
  const size_t rs = size_t(kv_heads) * D;  // elements between consecutive tokens
  const T* kbase = k + size_t(kstart) * rs + size_t(kv) * D;
  const T* vbase = v + size_t(kstart) * rs + size_t(kv) * D;

  auto load_block = [&](int id, BlockRegs<T>& R) {
    const int j0 = id * kBlock + wave * 16;
    const int jq = j0 + tok;
    if (jq <= t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) R.k[i].load(kbase + size_t(jq) * rs + 32 * i + 8 * r);
      if (CIS) R.cw = cis[(size_t(kstart) + jq) * kv_heads + kv];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) R.k[i].zero();
      R.cw = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jv = j0 + 4 * u + e;
      if (jv <= t) R.v[e].load(vbase + size_t(jv) * rs + 8 * o); else R.v[e].zero();
    }
  };

  auto compute_block = [&](int id, const BlockRegs<T>& R) {
    const bool qvalid = id * kBlock + wave * 16 + tok <= t;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if constexpr (kBF16) {
          const uint4 qv = *reinterpret_cast<const uint4*>(&q_s[h * (D / 2) + 16 * i + 4 * r]);
          const uint4 kk = reinterpret_cast<const Row8<bf16_t>&>(R.k[i]).r;
          s[h] = dot2_bf16(qv.x, kk.x, s[h]);
          s[h] = dot2_bf16(qv.y, kk.y, s[h]);
          s[h] = dot2_bf16(qv.z, kk.z, s[h]);
          s[h] = dot2_bf16(qv.w, kk.w, s[h]);
        } else {
          const float* qq = reinterpret_cast<const float*>(&q_s[h * D + 32 * i + 8 * r]);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[h] = fmaf(qq[e], R.k[i].f(e), s[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] += __shfl_xor(s[h], 1, kWave);
      s[h] += __shfl_xor(s[h], 2, kWave);
      s[h] = qvalid ? s[h] * scale_log2 : -INFINITY;
    }
    const float cw = CIS ? R.cw : 1.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], wave_max(s[h]));
      float alpha = 1.f, p = 0.f;
      if (mn != -INFINITY) {
        alpha = fast_exp2(m[h] - mn);
        p = fast_exp2(s[h] - mn) * cw;
      }
      l[h] = l[h] * alpha + p;
      m[h] = mn;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] *= alpha;
      if (r == 0) p_s[wave][tok][h] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pe[h] = p_s[wave][4 * u + e][h];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float vf = R.v[e].f(d);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][d] = fmaf(pe[h], vf, acc[h][d]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  BlockRegs<T> A, B;
  if (nv > 0) load_block(ids_s[0], A);
  for (int i = 0; i < nv; i += 2) {
    const int id0 = ids_s[i];
    const bool has1 = i + 1 < nv;
    const int id1 = has1 ? ids_s[i + 1] : 0;
    if (has1) load_block(id1, B);
    compute_block(id0, A);
    if (has1) {
      if (i + 2 < nv) load_block(ids_s[i + 2], A);
      compute_block(id1, B);
    }
  }

  // wave totals: l counted once per quad lane, acc summed over the 4 token quarters
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lw = wave_sum(l[h]) * 0.25f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc[h][d] += __shfl_xor(acc[h][d], 16, kWave);
      acc[h][d] += __shfl_xor(acc[h][d], 32, kWave);
    }
    if (lane == 0) {
      m_s[wave][h] = m[h];
      l_s[wave][h] = lw;
    }
    if (u == 0) {
#pragma unroll
      for (int d = 0; d < 8; ++d) acc_s[wave][h][8 * o + d] = acc[h][d];
    }
  }
  __syncthreads();

  const int n_split = SPLIT ? int(gridDim.x) : 1;
#pragma unroll
  for (int it = 0; it < (G * D + 255) / 256; ++it) {
    const int i = tid + 256 * it;
    if (i >= G * D) break;  // G = 1: 128 merge items for 256 threads
    const int h = i / D, d = i % D;
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = m_s[w][h];
      M = fmaxf(M, mw[w]);
    }
    float L = 0.f, Acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = fast_exp2(mw[w] - M);
        L += f * l_s[w][h];
        Acc += f * acc_s[w][h][d];
      }
    }
    if constexpr (SPLIT) {
      const size_t ps = unit * n_split + split;
      part_acc[(ps * G + h) * D + d] = Acc;
      if (d == 0) part_ml[ps * G + h] = make_float2(M, L);
    } else {
      store_f32(out + (unit * G + h) * D + d, L > 0.f ? Acc / L : 0.f);
      if (lse != nullptr && d == 0)
        lse[unit * G + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// bf16 variant on the matrix cores.  Per wave and block: the wave's 16 tokens
// against the group's query heads padded to 16 columns, S^T = K Q^T with four
// v_mfma_f32_16x16x32_bf16 (K rows straight from HBM in the A-operand layout,
// Q^T held in registers); lane (row r, column c) then holds the scores of tokens
// 4r..4r+3 for head c, so the softmax needs only in-lane work plus two lane
// swaps for the wave maximum; O^T += V^T P^T with eight v_mfma_f32_16x16x16_bf16
// takes P^T in exactly that layout (two packed conversions) and V^T from the
// V rows (below).  No LDS and no shuffles inside the block loop.  The running
// maximum is only raised when a block exceeds it by more than 2^8, so rescaling
// is rare.  Three waves per SIMD.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool CIS>
// Output dims are permuted across the eight O^T tiles: row c of tile n is dim
// 8c + n.  The A operand of tile n then needs, in lane (c16, r4), element n of
// dims 8 c16 .. 8 c16 + 7 of tokens 4 r4 .. 4 r4 + 3: four 16-byte loads of V
// rows per block instead of 32 two-byte gathers.
struct MfmaBlockRegs {
  uint4 k[4];   // A operand of S^T = K Q^T: token c16, dims 32i + 8 r4 .. +8
  uint4 v[4];   // V rows: token 4 r4 + e, dims 8 c16 .. 8 c16 + 7
  float cw[4];  // CIS of tokens 4 r4 + e
};

// LDS of the wave merge at the end of attend_staged_blocks.  Staged rows are
// padded to 80 floats: the merge reads lane c16 + 16w of rows 4n + r4, which
// then fall in distinct banks.
constexpr int kAccRow = kWave + 16;
struct MfmaAttnSmem {
  float m_s[4][16], l_s[4][16];
  float accx_s[4][32][kAccRow];  // [wave][tile element 4n + e][lane]
};

// Stage ids[s_begin, s_end) of one row that are valid for position t (id >= 0,
// block start <= t) into ids_s, in order; returns the count through nv_s (set
// by wave 0, read after the caller's barrier).
__device__ __forceinline__ void stage_ids(const int* ids, int s_begin, int s_end, int t,
                                          int* ids_s, int* nv_s) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) != 0) return;
  int base = 0;
  for (int s0 = s_begin; s0 < s_end; s0 += kWave) {
    const int sl = s0 + lane;
    const int id = sl < s_end ? ids[sl] : -1;
    const bool ok = id >= 0 && id * kBlock <= t;
    const unsigned long long mask = __ballot(ok);
    const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
    if (ok && pos < kMaxWgSlots) ids_s[pos] = id;
    base += __popcll(mask);
  }
  if (lane == 0) *nv_s = min(base, kMaxWgSlots);
}

// B operand of S^T = K Q^T: Q^T[dims 32i + 8 r4 .. +8][head c16].  Columns past
// G repeat head G-1: every step of the attention keeps the columns apart and
// none of theirs is written, so they need no zeroing (which would have to wait
// for the loads to land).
template <int G>
__device__ __forceinline__ void load_q_operand(const bf16_t* __restrict__ q, size_t unit,
                                               uint4 (&qb)[4]) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
  const bf16_t* qp = q + (unit * G + min(c16, G - 1)) * kHeadDim + 8 * r4;
#pragma unroll
  for (int i = 0; i < 4; ++i) qb[i] = ld16(qp + 32 * i);
}

// The G heads of `unit` (query position t of the sequence starting at kstart)
// attend to the nv staged block ids; the result is written as split `split` of
// n_split partial states (SPLIT) or as the output rows.  POOL: k and v are a
// block pool [units][pool_slots][64][128] and block ids_s[i] sits in slot
// slots_s[i] (the CIS values, when given, stay indexed by token).
template <int G, bool CIS, bool SPLIT, bool POOL = false>
__device__ __forceinline__ void attend_staged_blocks(
    MfmaAttnSmem& sm, const int* ids_s, int nv, const uint4 (&qb)[4],
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ cis,
    int kstart, int t, size_t unit, int kv, int kv_heads, float scale_log2, int split,
    int n_split, bf16_t* __restrict__ out, float* __restrict__ lse,
    float2* __restrict__ part_ml, float* __restrict__ part_acc,
    const int* slots_s = nullptr, int pool_slots = 0) {
  static_assert(G <= 16, "one MFMA column per query head");
  constexpr int D = kHeadDim;
  constexpr float kLazy = 8.f;  // log2-domain slack before the running max is raised
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  float (&m_s)[4][16] = sm.m_s;
  float (&l_s)[4][16] = sm.l_s;
  float (&accx_s)[4][32][kAccRow] = sm.accx_s;
  (void)tid;

  const size_t rs = POOL ? size_t(D) : size_t(kv_heads) * D;
  const bf16_t* kbase = POOL ? k + unit * size_t(pool_slots) * kBlock * D
                             : k + size_t(kstart) * rs + size_t(kv) * D;
  const bf16_t* vbase = POOL ? v + unit * size_t(pool_slots) * kBlock * D
                             : v + size_t(kstart) * rs + size_t(kv) * D;

  // Token rows past t are clamped to t: they lie inside the sequence (finite
  // data) and their probabilities are 0, so no per-load branches are needed.
  // Staged place i holds block ids_s[i]; in a pool, token j of that block is
  // row slots_s[i] * 64 + j - ids_s[i] * 64.
  auto load_block = [&](int i_st, MfmaBlockRegs<CIS>& R) {
    const int id = ids_s[i_st];
    const int j0 = id * kBlock + wave * 16;
    const int rb = POOL ? (slots_s[i_st] - id) * kBlock : 0;  // pool row of token j: j + rb
    const bf16_t* kr = kbase + size_t(min(j0 + c16, t) + rb) * rs + 8 * r4;
#pragma unroll
    for (int i = 0; i < 4; ++i) R.k[i] = ld16(kr + 32 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      R.v[e] = ld16(vbase + size_t(min(j0 + 4 * r4 + e, t) + rb) * rs + 8 * c16);
    if (CIS) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        R.cw[e] = cis[(size_t(kstart) + min(j0 + 4 * r4 + e, t)) * kv_heads + kv];
    }
  };

  float m_run = -INFINITY;  // running max of head c16 (same in the wave's 4 rows)
  float l_run = 0.f;        // this lane's share of the normaliser (its row's tokens)
  f32x4_t acc[8];           // O^T[dim 8 (4 r4 + e) + n][head c16]
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute_block = [&](int id, const MfmaBlockRegs<CIS>& R) {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.k[i]),
                                                     __builtin_bit_cast(bf16x8_t, qb[i]), sacc,
                                                     0, 0, 0);
    const int jrow = id * kBlock + wave * 16 + 4 * r4;
    float sv[4];
    float rmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = jrow + e <= t ? sacc[e] * scale_log2 : -INFINITY;
      rmax = fmaxf(rmax, sv[e]);
    }
    // wave max of head c16: rows pair up through the two lane swaps
    {
      auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
      rmax = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
      auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
      rmax = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
    }
    if (rmax > m_run + kLazy) {  // also true for the first block with a valid token
      const float alpha = fast_exp2(m_run - rmax);
      m_run = rmax;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = sv[e] == -INFINITY ? 0.f : fast_exp2(sv[e] - m_run);
      if (CIS) p[e] *= R.cw[e];
      l_run += p[e];
    }
    const bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
    const bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(__builtin_bit_cast(uint32_t, p01),
                                                              __builtin_bit_cast(uint32_t, p23)));
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      // element n of the four token rows: tokens 4 r4 .. 4 r4 + 3 of dim 8 c16 + n
      const uint32_t w0 = (&R.v[0].x)[n >> 1], w1 = (&R.v[1].x)[n >> 1];
      const uint32_t w2 = (&R.v[2].x)[n >> 1], w3 = (&R.v[3].x)[n >> 1];
      const uint32_t lo = (n & 1) ? (w0 >> 16) | (w1 & 0xFFFF0000u) : (w0 & 0xFFFFu) | (w1 << 16);
      const uint32_t hi = (n & 1) ? (w2 >> 16) | (w3 & 0xFFFF0000u) : (w2 & 0xFFFFu) | (w3 << 16);
      const s16x4_t va = __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[n], 0, 0, 0);
    }
  };

  MfmaBlockRegs<CIS> A, B;
  if (nv > 0) load_block(0, A);
  for (int i = 0; i < nv; i += 2) {
    const int id0 = ids_s[i];
    const bool has1 = i + 1 < nv;
    const int id1 = has1 ? ids_s[i + 1] : 0;
    if (has1) load_block(i + 1, B);
    compute_block(id0, A);
    if (has1) {
      if (i + 2 < nv) load_block(i + 2, A);
      compute_block(id1, B);
    }
  }

  // wave state of head c16: normaliser summed over the 4 rows
  {
    auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    float l2 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(l2), __float_as_uint(l2), false, false);
    l_run = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  }
  if (r4 == 0) {
    m_s[wave][c16] = m_run;
    l_s[wave][c16] = l_run;
  }
  // every wave holds the same tile layout: lane-minor staging is conflict-free
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) accx_s[wave][4 * n + e][lane] = acc[n][e];
  __syncthreads();

  // thread (wave w, r4, c16) merges head c16, dims 32w + 8 r4 .. +8 of the four
  // waves: in every wave's staged tiles these are rows 4n + r4 (n = 0..7) of
  // lane c16 + 16w; it writes them as one run
  float f[4], M = -INFINITY, L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = m_s[w][c16];
    M = fmaxf(M, f[w]);
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = (M == -INFINITY || f[w] == -INFINITY) ? 0.f : fast_exp2(f[w] - M);
    L += f[w] * l_s[w][c16];
  }
  const size_t ps = unit * n_split + split;
  float o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    o[n] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[n] += f[w] * accx_s[w][4 * n + r4][c16 + 16 * wave];
  }
  const int d0 = 32 * wave + 8 * r4;
  if (c16 < G) {
    if constexpr (SPLIT) {
      float* dst = part_acc + (ps * G + c16) * D + d0;
      *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
    } else if (part_acc != nullptr) {
      // unsplit rows may ask for float32 output rows (passed in part_acc)
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* dst = part_acc + (unit * G + c16) * D + d0;
      *reinterpret_cast<float4*>(dst) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16x2(L > 0.f ? o[2 * i] / L : 0.f, L > 0.f ? o[2 * i + 1] / L : 0.f);
      *reinterpret_cast<uint4*>(out + (unit * G + c16) * D + d0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  if (wave == 0 && r4 == 0 && c16 < G) {
    if constexpr (SPLIT) {
      part_ml[ps * G + c16] = make_float2(M, L);
    } else if (lse != nullptr) {
      lse[unit * G + c16] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

template <int G, bool CIS, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void selected_attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int* __restrict__ indices, int k_sel, const float* __restrict__ cis,
    bf16_t* __restrict__ out, float* __restrict__ lse, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int batch, int kv_heads, float scale_log2, int bpw,
    float2* __restrict__ part_ml, float* __restrict__ part_acc) {
  __shared__ MfmaAttnSmem sm;
  __shared__ int ids_s[kMaxWgSlots];
  __shared__ int nv_s;
  const int kv = blockIdx.y;
  const int row = SPLIT ? int(blockIdx.z) : int(blockIdx.x);
  const int split = SPLIT ? int(blockIdx.x) : 0;
  int b, t;
  attn_row_position(row, cu_q, cu_k, batch, b, t);
  const size_t unit = size_t(row) * kv_heads + kv;
  const int s_begin = split * bpw;
  const int s_end = SPLIT ? min(k_sel, s_begin + bpw) : k_sel;
  stage_ids(indices + unit * k_sel, s_begin, s_end, t, ids_s, &nv_s);
  uint4 qb[4];
  load_q_operand<G>(q, unit, qb);
  __syncthreads();
  attend_staged_blocks<G, CIS, SPLIT>(sm, ids_s, nv_s, qb, k, v, cis, cu_k[b], t, unit, kv,
                                      kv_heads, scale_log2, split, SPLIT ? int(gridDim.x) : 1,
                                      out, lse, part_ml, part_acc);
}

// Decode over a block pool (KV offload): like selected_attn_mfma_kernel with
// SPLIT, but the K/V rows of listed block indices[unit][p] come from pool slot
// slot_ids[unit][p] (the offload plan); a one-dimensional grid over (sequence,
// kv head, split).
template <int G, bool CIS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void pool_attn_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kpool,
    const bf16_t* __restrict__ vpool, const int* __restrict__ indices,
    const int* __restrict__ slot_ids, int k_sel, int pool_slots, const float* __restrict__ cis,
    const int* __restrict__ cu_k, int kv_heads, float scale_log2, int bpw,
    float2* __restrict__ part_ml, float* __restrict__ part_acc) {
  __shared__ MfmaAttnSmem sm;
  __shared__ int ids_s[kMaxWgSlots];
  __shared__ int slots_s[kMaxWgSlots];
  __shared__ int nv_s;
  // one-dimensional grid over (sequence, kv head, split), XCD-grouped as in the
  // resident decode step
  const int n_split = (k_sel + bpw - 1) / bpw;
  const int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  const int unit_i = m / n_split;
  const int split = m - unit_i * n_split, kv = unit_i % kv_heads, b = unit_i / kv_heads;
  const size_t unit = size_t(unit_i);
  uint4 qb[4];
  load_q_operand<G>(q, unit, qb);
  const int kstart = cu_k[b];
  const int t = cu_k[b + 1] - kstart - 1;
  const int s_begin = split * bpw, s_end = min(k_sel, s_begin + bpw);
  if (threadIdx.x < kWave) {
    const int p = s_begin + int(threadIdx.x);
    const int id = p < s_end ? indices[unit * k_sel + p] : -1;
    const int sl = p < s_end ? slot_ids[unit * k_sel + p] : -1;
    const bool ok = id >= 0 && id * kBlock <= t && sl >= 0 && sl < pool_slots;
    const unsigned long long m = __ballot(ok);
    const int pos = __popcll(m & ((1ull << threadIdx.x) - 1ull));
    if (ok) {
      ids_s[pos] = id;
      slots_s[pos] = sl;
    }
    if (threadIdx.x == 0) nv_s = __popcll(m);
  }
  __syncthreads();
  attend_staged_blocks<G, CIS, true, true>(sm, ids_s, nv_s, qb, kpool, vpool, cis, kstart, t,
                                           unit, kv, kv_heads, scale_log2, split, n_split,
                                           nullptr, nullptr, part_ml, part_acc, slots_s,
                                           pool_slots);
}

// Decode: score the blocks, select and attend in one launch.  Every workgroup
// of a (sequence, kv head) whose run of `bpw` places holds a free pick runs the
// same selection (identical inputs, so identical ids); a run of forced places
// only (the local window, or everything when all eligible blocks are chosen)
// takes its ids from the geometry and starts on its K/V at once.  Each split
// then attends to its run and writes a partial state; split 0 always selects
// and also writes the debug outputs.  One-dimensional grid over (sequence, kv
// head, split), in XCD-grouped order.
// MAXB bounds the blocks of a sequence: each thread keeps MAXB / 256 of them,
// so a smaller bound means less work in every step of the selection.
template <int G, bool CIS, int MAXB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void select_attn_kernel(
    const float* __restrict__ logits, const float2* __restrict__ part,
    const float* __restrict__ cisb, float cis_weight, const int* __restrict__ cu_k,
    const int* __restrict__ cu_c, int kv_heads, int nc_max, int ldc, int nb_max,
    int n_chunk_max, int ldb, int topk, int n_init, int n_local, int n_cand,
    float* __restrict__ block_scores, int* __restrict__ indices, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ cis,
    float scale_log2, int bpw, float2* __restrict__ part_ml, float* __restrict__ part_acc) {
  using Sel = SelCfg<256, MAXB>;
  __shared__ union {
    SelShared<256, MAXB> sel;
    MfmaAttnSmem att;
  } U;
  __shared__ int ids_s[kMaxWgSlots];
  __shared__ int nv_s;
  const int tid = threadIdx.x;
  // one-dimensional grid: the splits of one (sequence, kv head) run on one XCD,
  // which then reads the selection inputs of that unit into its L2 once
  const int n_split = (topk + bpw - 1) / bpw;
  const int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  const int unit_i = m / n_split;
  const int split = m - unit_i * n_split, kv = unit_i % kv_heads, b = unit_i / kv_heads;
  const size_t unit = size_t(unit_i);
  // the selection's inputs and the queries are in flight while the sequence
  // offsets arrive
  ScoreInputs<G, 256, MAXB> sin;
  load_score_inputs(sin, logits, part, cisb, unit, n_chunk_max, ldc, ldb);
  uint4 qb[4];
  load_q_operand<G>(q, unit, qb);
  const int kstart = cu_k[b];
  const int len = cu_k[b + 1] - kstart;
  const int t = len - 1;
  const int nb = min(nb_max, (len + kBlock - 1) / kBlock);
  const int nvis = min(cu_c[b + 1] - cu_c[b], full_windows_dev(len));
  const bool lead = split == 0;
  const SelGeom g = sel_geometry(t, nb, topk, n_init, n_local, n_cand);
  const int s_begin = split * bpw, s_end = min(topk, s_begin + bpw);
  // A split whose places hold no free pick knows its ids from the geometry
  // alone and skips the selection; the lead split always selects, since it
  // writes the row's indices and block scores.  (Uniform per workgroup.)
  const bool known = !lead && (g.free_mark != 2 || s_end <= g.f_init || s_begin >= g.f_init + g.kf);
  if (known) {
    if (tid < kWave) {
      const int p = s_begin + tid;
      const int id = p < s_end ? forced_id_at(g, p) : -1;
      if (id >= 0) ids_s[tid] = id;  // ids are ascending, so the valid ones are a prefix
      const int n = __popcll(__ballot(id >= 0));
      if (tid == 0) nv_s = n;
    }
  } else {
    float sc[Sel::kPer], scc[Sel::kPer];
    block_scores_from_logits<G, 256, MAXB>(U.sel, sc, scc, n_cand > 0, sin, logits, cisb,
                                           cis_weight, unit, nvis, nb, ldc, nb_max, nc_max,
                                           lead ? block_scores : nullptr, nullptr);
    int* irow = indices != nullptr && lead ? indices + unit * topk : nullptr;
    // every chosen id is eligible (start <= t): the split's ids go straight to
    // its slots, the lead's also to the row's indices
    const int total = topk_select<256, MAXB>(U.sel, sc, scc, n_cand, g, topk, [&](int pos, int id) {
      if (pos >= s_begin && pos < s_end) ids_s[pos - s_begin] = id;
      if (irow != nullptr) irow[pos] = id;
    });
    if (irow != nullptr)
      for (int i = total + tid; i < topk; i += 256) irow[i] = -1;
    if (tid == 0) nv_s = max(0, min(total, s_end) - s_begin);
  }
  __syncthreads();
  attend_staged_blocks<G, CIS, true>(U.att, ids_s, nv_s, qb, k, v, cis, kstart, t, unit, kv,
                                     kv_heads, scale_log2, split, n_split, nullptr,
                                     nullptr, part_ml, part_acc);
}

// Merge the per-split partial states of one (row, kv head, query head): a
// one-dimensional grid over (unit, query head) in XCD-grouped order, like the
// decode splits that wrote them; one thread per output dim.
template <typename T>
__global__ __launch_bounds__(kHeadDim) void combine_kernel(const float2* __restrict__ part_ml,
                                                           const float* __restrict__ part_acc,
                                                           T* __restrict__ out,
                                                           float* __restrict__ lse, int n_split,
                                                           int G) {
  constexpr int D = kHeadDim;
  __shared__ float f_s[kMaxSplits];
  __shared__ float ML_s[2];
  const int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  const size_t unit = size_t(m / G);
  const int h = m - int(unit) * G, d = threadIdx.x;
  // every load first: the (max, sum) pair of split d and this dim of every split
  const float2 ml0 = part_ml[(unit * n_split + min(d, n_split - 1)) * G + h];
  const float* src = part_acc + (unit * n_split * G + h) * D + d;
  const size_t stride = size_t(G) * D;
  float x[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) x[sp] = sp < n_split ? src[sp * stride] : 0.f;
  // max and normaliser over the splits (n_split <= 64: one wave holds them all)
  if (d < kWave) {
    const float mx = d < n_split ? ml0.x : -INFINITY;
    const float M = wave_max(mx);
    const float f = (d < n_split && M != -INFINITY && mx != -INFINITY) ? fast_exp2(mx - M) : 0.f;
    const float L = wave_sum(f * (d < n_split ? ml0.y : 0.f));
    f_s[d] = f;
    if (d == 0) {
      ML_s[0] = M;
      ML_s[1] = L;
    }
  }
  __syncthreads();
  const float L = ML_s[1];
  float accv = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < n_split) accv += f_s[sp] * x[sp];
  store_f32(out + (unit * G + h) * D + d, L > 0.f ? accv / L : 0.f);
  if (lse != nullptr && d == 0) lse[unit * G + h] = L > 0.f ? (ML_s[0] + __log2f(L)) * kLn2 : -INFINITY;
}

// --------------------------------------------------------------------------- host

int attn_split_blocks(int batch, int kv_heads, int k_sel) {
  // enough workgroups to give every CU one, at most 8 blocks each, <= kMaxSplits
  // splits.  More splits spread the block loads wider but every split of a
  // fused decode row repeats the row's selection (one workgroup per CU measured
  // fastest: 16 units of 64 blocks at 4 blocks per split)
  const int units = batch * kv_heads;
  int bpw = 8;
  while (bpw > 1 && units * ((k_sel + bpw - 1) / bpw) < 256) bpw >>= 1;
  while ((k_sel + bpw - 1) / bpw > kMaxSplits) bpw <<= 1;
  return bpw;
}

size_t attn_ws_bytes(int rows_total, int kv_heads, int group, int k_sel, int decode) {
  if (!decode) return 0;
  const size_t units = size_t(rows_total) * kv_heads;
  const int bpw = attn_split_blocks(rows_total, kv_heads, k_sel);
  const size_t n_split = (size_t(k_sel) + bpw - 1) / bpw;
  size_t bytes = ((units * n_split * group * sizeof(float2)) + 255) & ~size_t(255);
  bytes += ((units * n_split * group * kHeadDim * sizeof(float)) + 255) & ~size_t(255);
  return bytes;
}

AttnWs attn_ws_carve(void* base, int rows_total, int kv_heads, int group, int k_sel, int decode) {
  AttnWs ws{nullptr, nullptr};
  if (!decode) return ws;
  const size_t units = size_t(rows_total) * kv_heads;
  const int bpw = attn_split_blocks(rows_total, kv_heads, k_sel);
  const size_t n_split = (size_t(k_sel) + bpw - 1) / bpw;
  char* p = static_cast<char*>(base);
  ws.part_ml = reinterpret_cast<float2*>(p);
  p += (units * n_split * group * sizeof(float2) + 255) & ~size_t(255);
  ws.part_acc = reinterpret_cast<float*>(p);
  return ws;
}

template <typename T>
using AttnKernelFn = void (*)(const T*, const T*, const T*, const int*, int, const float*, T*,
                              float*, const int*, const int*, int, int, float, int, float2*,
                              float*);

// bf16 runs on the matrix cores; float32 on the vector ALUs.
template <int G, typename T, bool CIS, bool SPLIT>
static AttnKernelFn<T> attn_kernel_for() {
  if constexpr (sizeof(T) == 2) return selected_attn_mfma_kernel<G, CIS, SPLIT>;
  else return selected_attn_valu_kernel<G, T, CIS, SPLIT>;
}

template <int G, typename T, bool CIS>
static hipError_t launch_attn_g(const void* q, const void* k, const void* v, const int* indices,
                                int k_sel, const float* cis, void* out, float* lse,
                                const int* cu_q, const int* cu_k, int batch, int rows_total,
                                int kv_heads, float scale_log2, const AttnWs& ws, hipStream_t s,
                                float* out_f32) {
  if (rows_total == 0 || k_sel == 0) return hipSuccess;
  if (cu_q == nullptr) {
    const int bpw = attn_split_blocks(rows_total, kv_heads, k_sel);
    const int n_split = (k_sel + bpw - 1) / bpw;
    hipError_t e = launch_kernel(
        kKindAttn, attn_kernel_for<G, T, CIS, true>(), dim3(n_split, kv_heads, rows_total),
        dim3(256), s, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
        indices, k_sel, cis, static_cast<T*>(out), lse, cu_q, cu_k, batch, kv_heads, scale_log2,
        bpw, ws.part_ml, ws.part_acc);
    if (e != hipSuccess) return e;
    return launch_kernel(kKindCombine, combine_kernel<T>, dim3(rows_total * kv_heads * G),
                         dim3(kHeadDim), s, static_cast<const float2*>(ws.part_ml),
                         static_cast<const float*>(ws.part_acc), static_cast<T*>(out), lse,
                         n_split, G);
  }
  return launch_kernel(kKindAttn, attn_kernel_for<G, T, CIS, false>(),
                       dim3(rows_total, kv_heads, 1), dim3(256), s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), indices, k_sel, cis,
                       static_cast<T*>(out), lse, cu_q, cu_k, batch, kv_heads, scale_log2, k_sel,
                       static_cast<float2*>(nullptr), out_f32);
}

template <typename T, bool CIS>
static hipError_t launch_attn_t(int G, const void* q, const void* k, const void* v,
                                const int* idx, int k_sel, const float* cis, void* out, float* lse,
                                const int* cu_q, const int* cu_k, int batch, int rows,
                                int kvh, float sl2, const AttnWs& ws, hipStream_t s,
                                float* out_f32) {
  switch (G) {
    case 1: return launch_attn_g<1, T, CIS>(q, k, v, idx, k_sel, cis, out, lse, cu_q, cu_k, batch, rows, kvh, sl2, ws, s, out_f32);
    case 2: return launch_attn_g<2, T, CIS>(q, k, v, idx, k_sel, cis, out, lse, cu_q, cu_k, batch, rows, kvh, sl2, ws, s, out_f32);
    case 4: return launch_attn_g<4, T, CIS>(q, k, v, idx, k_sel, cis, out, lse, cu_q, cu_k, batch, rows, kvh, sl2, ws, s, out_f32);
    case 8: return launch_attn_g<8, T, CIS>(q, k, v, idx, k_sel, cis, out, lse, cu_q, cu_k, batch, rows, kvh, sl2, ws, s, out_f32);
    case 16: return launch_attn_g<16, T, CIS>(q, k, v, idx, k_sel, cis, out, lse, cu_q, cu_k, batch, rows, kvh, sl2, ws, s, out_f32);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_selected_attn(const void* q, const void* k, const void* v, int bf16,
                                const int* indices, int k_sel, const float* cis, void* out,
                                float* lse, const int* cu_q, const int* cu_k, int batch,
                                int rows_total, int heads, int kv_heads, float scale_log2,
                                const AttnWs& ws, hipStream_t s, float* out_f32) {
  const int G = heads / kv_heads;
  if (!bf16) out_f32 = nullptr;  // float32 inputs write float32 rows to out already
  if (bf16) {
    if (cis) return launch_attn_t<bf16_t, true>(G, q, k, v, indices, k_sel, cis, out, lse, cu_q, cu_k, batch, rows_total, kv_heads, scale_log2, ws, s, out_f32);
    return launch_attn_t<bf16_t, false>(G, q, k, v, indices, k_sel, cis, out, lse, cu_q, cu_k, batch, rows_total, kv_heads, scale_log2, ws, s, out_f32);
  }
  if (cis) return launch_attn_t<float, true>(G, q, k, v, indices, k_sel, cis, out, lse, cu_q, cu_k, batch, rows_total, kv_heads, scale_log2, ws, s, out_f32);
  return launch_attn_t<float, false>(G, q, k, v, indices, k_sel, cis, out, lse, cu_q, cu_k, batch, rows_total, kv_heads, scale_log2, ws, s, out_f32);
}

template <int G, bool CIS>
static hipError_t launch_select_attn_g(const DecodeScoresArgs& a, const void* k, const void* v,
                                       const float* cis_values, void* out, const AttnWs& ws,
                                       hipStream_t s) {
  const ScoreDims d = score_dims(a.max_seqlen_k);
  const int bpw = attn_split_blocks(a.batch, a.kv_heads, a.topk);
  const int n_split = (a.topk + bpw - 1) / bpw;
  const float* cisb = a.cis_pooled != nullptr ? a.ws.cisb : nullptr;
  auto kern = d.nb_max <= kFusedSmallBlocks ? select_attn_kernel<G, CIS, kFusedSmallBlocks>
             : d.nb_max <= kFusedMidBlocks  ? select_attn_kernel<G, CIS, kFusedMidBlocks>
                                            : select_attn_kernel<G, CIS, kFusedMaxBlocks>;
  hipError_t e = launch_kernel(
      kKindAttn, kern, dim3(n_split * a.kv_heads * a.batch), dim3(256), s,
      static_cast<const float*>(a.ws.logits), static_cast<const float2*>(a.ws.part), cisb,
      a.cis_weight, a.cu_k, a.cu_c, a.kv_heads, d.nc_max, d.ldc, d.nb_max, d.n_chunk_max, d.ldb,
      a.topk, a.n_init, a.n_local, a.n_cand, a.block_scores, a.indices, static_cast<const bf16_t*>(a.q),
      static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), cis_values, a.scale_log2, bpw,
      ws.part_ml, ws.part_acc);
  if (e != hipSuccess) return e;
  return launch_kernel(kKindCombine, combine_kernel<bf16_t>, dim3(a.batch * a.kv_heads * G),
                       dim3(kHeadDim), s, static_cast<const float2*>(ws.part_ml),
                       static_cast<const float*>(ws.part_acc), static_cast<bf16_t*>(out),
                       static_cast<float*>(nullptr), n_split, G);
}

template <int G, bool CIS>
static hipError_t launch_pool_attn_g(const void* q, const OffloadArgs& a, const float* cis_values,
                                     void* out, float scale_log2, const AttnWs& ws,
                                     hipStream_t s) {
  const int batch = a.units / a.kv_heads;
  const int bpw = attn_split_blocks(batch, a.kv_heads, a.k_sel);
  const int n_split = (a.k_sel + bpw - 1) / bpw;
  hipError_t e = launch_kernel(
      kKindAttn, pool_attn_kernel<G, CIS>, dim3(n_split * a.units), dim3(256), s,
      static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(a.kpool),
      static_cast<const bf16_t*>(a.vpool), a.indices, static_cast<const int*>(a.slot_ids),
      a.k_sel, a.pool_slots, cis_values, a.cu_k, a.kv_heads, scale_log2, bpw, ws.part_ml,
      ws.part_acc);
  if (e != hipSuccess) return e;
  return launch_kernel(kKindCombine, combine_kernel<bf16_t>, dim3(a.units * G), dim3(kHeadDim), s,
                       static_cast<const float2*>(ws.part_ml),
                       static_cast<const float*>(ws.part_acc), static_cast<bf16_t*>(out),
                       static_cast<float*>(nullptr), n_split, G);
}

template <bool CIS>
static hipError_t launch_pool_attn_c(int G, const void* q, const OffloadArgs& a,
                                     const float* cis_values, void* out, float scale_log2,
                                     const AttnWs& ws, hipStream_t s) {
  switch (G) {
    case 1: return launch_pool_attn_g<1, CIS>(q, a, cis_values, out, scale_log2, ws, s);
    case 2: return launch_pool_attn_g<2, CIS>(q, a, cis_values, out, scale_log2, ws, s);
    case 4: return launch_pool_attn_g<4, CIS>(q, a, cis_values, out, scale_log2, ws, s);
    case 8: return launch_pool_attn_g<8, CIS>(q, a, cis_values, out, scale_log2, ws, s);
    case 16: return launch_pool_attn_g<16, CIS>(q, a, cis_values, out, scale_log2, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pool_attn(const void* q, const OffloadArgs& a, const float* cis_values,
                            void* out, int heads, float scale_log2, const AttnWs& ws,
                            hipStream_t s) {
  const int G = heads / a.kv_heads;
  if (cis_values != nullptr)
    return launch_pool_attn_c<true>(G, q, a, cis_values, out, scale_log2, ws, s);
  return launch_pool_attn_c<false>(G, q, a, cis_values, out, scale_log2, ws, s);
}

template <bool CIS>
static hipError_t launch_select_attn_c(int G, const DecodeScoresArgs& a, const void* k,
                                       const void* v, const float* cis_values, void* out,
                                       const AttnWs& ws, hipStream_t s) {
  switch (G) {
    case 1: return launch_select_attn_g<1, CIS>(a, k, v, cis_values, out, ws, s);
    case 2: return launch_select_attn_g<2, CIS>(a, k, v, cis_values, out, ws, s);
    case 4: return launch_select_attn_g<4, CIS>(a, k, v, cis_values, out, ws, s);
    case 8: return launch_select_attn_g<8, CIS>(a, k, v, cis_values, out, ws, s);
    case 16: return launch_select_attn_g<16, CIS>(a, k, v, cis_values, out, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_select_attn(const DecodeScoresArgs& a, const void* k, const void* v,
                              const float* cis_values, void* out, const AttnWs& ws,
                              hipStream_t s) {
  const int G = a.heads / a.kv_heads;
  if (cis_values != nullptr) return launch_select_attn_c<true>(G, a, k, v, cis_values, out, ws, s);
  return launch_select_attn_c<false>(G, a, k, v, cis_values, out, ws, s);
}

}  // namespace nsa
