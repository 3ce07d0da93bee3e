// Selected attention over prefill rows, key-block stationary.
//
// What is computed is the selected attention of TileLang NSA, section 2: query
// row t of a sequence attends to the 64-token blocks its index row lists (block
// id i starts at token 64 i and counts when 0 <= 64 i <= t; keys past t are
// masked), the G query heads of one KV group sharing the blocks; in CIS mode
// (NOSA-1B core components, decode stage) every probability is scaled by its
// key's CIS value and the normaliser is the same sum over all-ones values.
//
// The row-by-row kernel gathers 64 K and V rows per listed block for every
// (row, KV head): with uniform block choices no two rows share a block, so its
// bytes come from L2 and the Infinity Cache, not from the matrix cores' reuse.
// Here the roles are swapped:
//
// block_partial_kernel -- one workgroup per (sequence, KV head, chunk of 1024
//   query rows, 64-key block).  It builds the block's matrix-core operands
//   once, in LDS (K in the A layout of S^T = K Q^T, V^T in the A layout of
//   O^T = V^T P^T), scans the chunk's index rows for the rows that list the
//   block (and at which place), and walks those rows in tiles of 16 query
//   vectors (a query vector is one (row, head) pair: 16/G rows of G heads), one
//   tile per wave at a time, so a tile costs its q rows in, 32
//   v_mfma_f32_16x16x32_bf16, and its partial state out: the block's
//   unnormalised output in bf16 plus (max, sum) in fp32, at the row's place.
// block_merge_kernel -- per (row, head): the partial states of the row's valid
//   places combined with the usual log-sum-exp weights.
//
// Precision is that of the row-by-row kernel: bf16 probabilities enter the
// matrix cores, fp32 sums (the normaliser sums the fp32 probabilities); each
// partial output is rounded to bf16 once more (2^-9 relative) before the
// merge.
#include <climits>

#include "common.h"
#include "launch.h"

namespace nsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) accesses of the partial states: written once, read
// once, so they bypass L2 allocation and leave it to the reused rows.
__device__ __forceinline__ void stream_store(bf16_t* p, uint4 x) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x), reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void stream_store(float* p, float x) { __builtin_nontemporal_store(x, p); }
__device__ __forceinline__ uint4 stream_load(const bf16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

constexpr int kScanRows = 1024;       // query rows one workgroup scans for its block
constexpr int kLdsRow = kHeadDim + 8; // bf16 per staged K/V row (272 B)
constexpr int kMaxPlaces = 64;        // index places per row (place fits 6 bits)
constexpr int kMergeBatch = 8;        // places whose loads the merge keeps in flight together

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t x = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, x);
}

__device__ __forceinline__ f32x16_t mfma32x32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// max / sum over lanes l and l ^ 32 (one column of a 32x32 accumulator)
__device__ __forceinline__ float pair_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// The block's matrix-core operands are the same for the four waves, so they are
// built once per workgroup and kept in LDS in lane order (lane-contiguous 16-byte
// reads, free of bank conflicts), for 32x32x16 bf16 tiles: operand lane l holds
// row (column) l % 32 at k indices 8 (l / 32) .. +7, and accumulator j of lane l
// is row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.  The k index of a product
// is summed over, so any fixed assignment of dims (keys) to it serves, as long as
// both operands use the same one:
//   kop[x][s][lane]: A of S^T = K Q^T for keys 32 x .. +31, step s: key
//     32 x + lane % 32, dims 64 (lane / 32) + 8 s .. +7 (the q operand of lane l
//     holds the same dims of its query vector);
//   vop[n][m][lane]: A of O^T += V^T P^T for output tile n, key step m: row
//     rho = lane % 32 is dim 32 n + f(rho), f(8 a + 4 g + b) = 16 (a / 2) + 8 g +
//     4 (a % 2) + b, and k index u of lane half g = lane / 32 is key
//     16 m + 8 (u / 4) + 4 g + u % 4.
// A lane's score accumulators j = 8 (m % 2) .. +7 of key half m / 2 are then
// exactly its k indices of P^T for key step m, and its output accumulators
// j = 8 i .. 8 i + 7 of tile n are the eight consecutive dims
// 32 n + 16 i + 8 (lane / 32) .. +7.
struct PartialLds {
  uint4 kop[2][8][64];
  uint4 vop[4][4][64];
  float cisw[kBlock];        // CIS of the block's keys (CIS mode)
  uint16_t list[kScanRows];  // (row in chunk << 6) | place
  int n_list;
};

// Append to the list the rows that list block `blk`, each at the first place
// holding it.  Vector form (k_sel a multiple of 4 and a 16-byte aligned array,
// so every index row is 16-byte aligned): P lanes per index row, 4 ids per lane, all of a batch's loads in
// flight together.
template <int P, typename Lds>
__device__ __forceinline__ void scan_rows_vec(Lds& sm, const int* __restrict__ indices,
                                              int k_sel, int kv_heads, int kv, int q0, int r_lo,
                                              int r_first, int r_hi, int blk, int wave, int lane) {
  constexpr int RPI = 64 / P;       // rows per wave instruction
  constexpr int kBatch = 16;        // loads in flight per lane
  const int seg = lane % P, gbase = lane & ~(P - 1);
  const int n_inst = (r_hi - r_first + 4 * RPI - 1) / (4 * RPI);
  for (int j0 = 0; j0 < n_inst; j0 += kBatch) {
    int4 idv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int r = r_first + ((j0 + j) * 4 + wave) * RPI + lane / P;
      const bool ok = j0 + j < n_inst && r < r_hi && 4 * seg < k_sel;
      const int* row = indices + (size_t(q0 + min(r, r_hi - 1)) * kv_heads + kv) * k_sel;
      idv[j] = ok ? *reinterpret_cast<const int4*>(row + 4 * seg) : make_int4(-1, -1, -1, -1);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j0 + j >= n_inst) break;  // the same for the whole wave
      const int r = r_first + ((j0 + j) * 4 + wave) * RPI + lane / P;
      const int4 x = idv[j];
      const int u = x.x == blk ? 0 : x.y == blk ? 1 : x.z == blk ? 2 : x.w == blk ? 3 : -1;
      const unsigned long long hit = __ballot(u >= 0);
      const unsigned long long grp = (hit >> gbase) & ((1ull << P) - 1ull);
      const bool writer = u >= 0 && (grp & ((1ull << seg) - 1ull)) == 0ull;
      const unsigned long long wmask = __ballot(writer);
      int base = 0;
      if (lane == 0 && wmask != 0ull) base = atomicAdd(&sm.n_list, __popcll(wmask));
      base = __shfl(base, 0);
      if (writer)
        sm.list[base + __popcll(wmask & ((1ull << lane) - 1ull))] = uint16_t(((r - r_lo) << 6) | (4 * seg + u));
    }
  }
}

// Scalar form for any k_sel: one thread per index row.
template <typename Lds>
__device__ __forceinline__ void scan_rows_scalar(Lds& sm, const int* __restrict__ indices,
                                                 int k_sel, int kv_heads, int kv, int q0, int r_lo,
                                                 int r_first, int r_hi, int blk, int tid, int lane) {
  for (int r0 = r_first; r0 < r_hi; r0 += 256) {
    const int r = r0 + tid;
    int place = -1;
    if (r < r_hi) {
      const int* ids = indices + (size_t(q0 + r) * kv_heads + kv) * k_sel;
      for (int p0 = 0; p0 < k_sel; p0 += 16) {
        int idv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) idv[u] = p0 + u < k_sel ? ids[p0 + u] : -1;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (place < 0 && idv[u] == blk) place = p0 + u;
      }
    }
    const unsigned long long mask = __ballot(place >= 0);
    int base = 0;
    if (lane == 0 && mask != 0ull) base = atomicAdd(&sm.n_list, __popcll(mask));
    base = __shfl(base, 0);
    if (place >= 0)
      sm.list[base + __popcll(mask & ((1ull << lane) - 1ull))] = uint16_t(((r - r_lo) << 6) | place);
  }
}

template <typename Lds>
__device__ __forceinline__ void scan_rows(Lds& sm, const int* __restrict__ indices, int k_sel,
                                          int kv_heads, int kv, int q0, int r_lo, int r_first,
                                          int r_hi, int blk) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if ((k_sel & 3) == 0 && (reinterpret_cast<uintptr_t>(indices) & 15) == 0) {
    const int lanes = k_sel / 4;
    if (lanes <= 1) scan_rows_vec<1>(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk, wave, lane);
    else if (lanes <= 2) scan_rows_vec<2>(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk, wave, lane);
    else if (lanes <= 4) scan_rows_vec<4>(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk, wave, lane);
    else if (lanes <= 8) scan_rows_vec<8>(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk, wave, lane);
    else scan_rows_vec<16>(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk, wave, lane);
  } else {
    scan_rows_scalar(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk, tid, lane);
  }
}

// The (sequence, KV head, row chunk, block) of a workgroup of a one-dimensional
// grid in XCD-grouped order (the blocks of one row chunk run together on one
// XCD and share its query rows and index rows in L2), and the chunk's rows.
struct BlockUnit {
  int blk, kv, b, kstart, L, q0, off, r_lo, r_hi, r_first;
};
__device__ __forceinline__ BlockUnit block_unit(const int* __restrict__ cu_q,
                                                const int* __restrict__ cu_k, int kv_heads,
                                                int nb_max, int n_chunk) {
  BlockUnit u;
  int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  u.blk = m % nb_max;
  m /= nb_max;
  const int chunk = m % n_chunk;
  m /= n_chunk;
  u.kv = m % kv_heads;
  u.b = m / kv_heads;
  u.kstart = cu_k[u.b];
  u.L = cu_k[u.b + 1] - u.kstart;
  u.q0 = cu_q[u.b];
  const int Lq = cu_q[u.b + 1] - u.q0;
  u.off = u.L - Lq;  // query row r of the sequence sits at position off + r
  u.r_lo = chunk * kScanRows;
  u.r_hi = min(Lq, u.r_lo + kScanRows);
  u.r_first = max(u.r_lo, kBlock * u.blk - u.off);  // rows that can list the block
  return u;
}

// Valid places of one index row for position t, as a bit mask: id >= 0, block
// start <= t, and no earlier place holding the same id.  Lane `sub` of a group
// of 16 lanes (the lanes of one query vector, `grp` its first lane) checks
// places sub, sub + 16, ... and compares them with the earlier places through
// the group; every lane of the group gets the whole mask.
__device__ __forceinline__ unsigned long long valid_places(const int* __restrict__ ids, int k_sel,
                                                          int t, int sub, int grp) {
  const int rounds = (k_sel + 15) >> 4;
  int myid[kMaxPlaces / 16];
#pragma unroll
  for (int u = 0; u < kMaxPlaces / 16; ++u) myid[u] = 16 * u + sub < k_sel ? ids[16 * u + sub] : -1;
  unsigned long long valid = 0ull;
#pragma unroll
  for (int u = 0; u < kMaxPlaces / 16; ++u) {
    if (u >= rounds) break;
    bool ok = myid[u] >= 0 && myid[u] <= t / kBlock;
#pragma unroll
    for (int w = 0; w <= u; ++w)
      for (int j = 0; j < 16; ++j) {
        const int other = __shfl(myid[w], grp + j);
        if (16 * w + j < 16 * u + sub && other == myid[u]) ok = false;
      }
    valid |= ((__ballot(ok) >> grp) & 0xFFFFull) << (16 * u);
  }
  return valid;
}

// Grid: one dimension over (sequence, KV head, row chunk, block) in XCD-grouped
// order, so the blocks of one row chunk run together on one XCD and share its
// query rows and index rows in L2.
//
// Partial states: pml[(row * k_sel + place) * heads + head] = (max, sum) in the
// log2 domain; the unnormalised bf16 outputs of the G heads of one (row, place,
// KV head) share the region of G * 128 values at
// po[((row * k_sel + place) * heads + kv * G) * 128 ..], in which dims
// 8 p .. 8 p + 7 of head hg sit at (p / 2) * 16 G + 16 hg + 8 (p % 2): one store
// instruction of a tile then writes 32 G contiguous bytes per list entry.
template <int G, bool CIS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void block_partial_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int* __restrict__ indices, int k_sel, const float* __restrict__ cis,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int kv_heads, int nb_max,
    int n_chunk, float scale_log2, bf16_t* __restrict__ po, float2* __restrict__ pml) {
  constexpr int E = 32 / G;  // list entries per tile of 32 query vectors
  constexpr int D = kHeadDim;
  __shared__ PartialLds sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, g = lane >> 5;

  const BlockUnit U = block_unit(cu_q, cu_k, kv_heads, nb_max, n_chunk);
  const int blk = U.blk, kv = U.kv, kstart = U.kstart, L = U.L, q0 = U.q0, off = U.off;
  const int r_lo = U.r_lo, r_hi = U.r_hi, r_first = U.r_first;
  if (r_first >= r_hi || kBlock * blk >= L) return;  // the same for the whole workgroup
  const int heads = kv_heads * G;

  // The block's operands straight from K and V (rows past the sequence end
  // repeat its last row: finite data, masked below since they lie past every
  // row's position), requested before the index scan so both are in flight
  // together.  Waves 0 and 1 load K (16-byte piece x = 128 i + tid is key x / 16,
  // dims 8 (x % 16) ..); waves 2 and 3 load V, thread t = tid - 128 taking dims
  // 8 (t % 16) .. +7 of the eight keys of step t / 32, lane half (t / 16) % 2, and
  // transposing them in registers.
  if (tid == 0) sm.n_list = 0;
  uint4 ld[8];
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = k + size_t(kstart) * rs + size_t(kv) * D;
  const bf16_t* vb = v + size_t(kstart) * rs + size_t(kv) * D;
  if (wave < 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int x = 128 * i + tid;
      ld[i] = ld16(kb + size_t(min(kBlock * blk + (x >> 4), L - 1)) * rs + 8 * (x & 15));
    }
  } else {
    const int t = tid - 128, m = t >> 5, gh = (t >> 4) & 1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = 16 * m + 8 * (u >> 2) + 4 * gh + (u & 3);
      ld[u] = ld16(vb + size_t(min(kBlock * blk + key, L - 1)) * rs + 8 * (t & 15));
    }
  }
  if (CIS && tid < kBlock) sm.cisw[tid] = cis[size_t(kstart + min(kBlock * blk + tid, L - 1)) * kv_heads + kv];
  __syncthreads();  // n_list = 0 seen by every wave
  scan_rows(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk);
  if (wave < 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int x = 128 * i + tid, key = x >> 4, pc = x & 15;
      sm.kop[key >> 5][pc & 7][(key & 31) + 32 * (pc >> 3)] = ld[i];
    }
  } else {
    // dims 8 (t % 16) + c = 32 n + 16 i + 8 gp + c are rows 8 (2 i + c / 4) + 4 gp + c % 4 of tile n
    const int t = tid - 128, m = t >> 5, gh = (t >> 4) & 1, db = t & 15;
    const int n = db >> 2, i = (db >> 1) & 1, gp = db & 1;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t a = (&ld[2 * x].x)[c >> 1], b = (&ld[2 * x + 1].x)[c >> 1];
        w[x] = (c & 1) ? (a >> 16) | (b & 0xFFFF0000u) : (a & 0xFFFFu) | (b << 16);
      }
      const int rho = 8 * (2 * i + (c >> 2)) + 4 * gp + (c & 3);
      sm.vop[n][m][rho + 32 * gh] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __syncthreads();
  const int n_list = sm.n_list;
  const int n_tiles = (n_list + E - 1) / E;
  if (wave >= n_tiles) return;  // no barrier below

  const int ent = c32 / G, hg = c32 % G;
  const int key0 = kBlock * blk + 4 * g;  // key of score j of half x: key0 + 32 x + 8 (j / 4) + j % 4
  const int last_key = kBlock * blk + kBlock - 1;
  // the log2-domain scale (positive) is applied inside one fma per score:
  // p = exp2(c s - c m) with m the raw maximum
  const float c = scale_log2;
  // chunk bases (uniform) and per-lane byte offsets below them, which fit 32 bits
  // for every shape the host admits
  const char* qbase = reinterpret_cast<const char*>(q + size_t(q0 + r_lo) * heads * D);
  char* pbase = reinterpret_cast<char*>(po + size_t(q0 + r_lo) * k_sel * heads * D);
  char* mbase = reinterpret_cast<char*>(pml + size_t(q0 + r_lo) * k_sel * heads);
  const uint32_t q_lane = uint32_t(((kv * G + hg) * D + 64 * g) * 2);
  const uint32_t p_lane = uint32_t((kv * G * D + 16 * hg + 8 * g) * 2);
  const uint32_t m_lane = uint32_t((kv * G + hg) * 8 + 4 * g);

  // One tile: this lane's query vector c32 (entry c32 / G of the tile, head
  // c32 % G): its list code, its position and its q operand.  A slot past the
  // list repeats the last entry: it computes that entry's values again and
  // stores the same bytes at the same addresses, so every store below is
  // unconditional.
  struct Tile {
    int code, t;
    uint4 q[8];
  };
  // tiles past the wave's last are clamped to the last one: the prefetch then
  // needs no branch, so its loads land straight in the registers that use them
  auto fetch = [&](int tile, Tile& T) {
    tile = min(tile, n_tiles - 1);
    T.code = sm.list[min(tile * E + ent, n_list - 1)];
    T.t = off + r_lo + (T.code >> 6);
    const char* qp = qbase + (uint32_t(T.code >> 6) * uint32_t(heads * D * 2) + q_lane);
#pragma unroll
    for (int s = 0; s < 8; ++s) T.q[s] = ld16(qp + 16 * s);
  };

  // One tile: the scores, then the next tile's q rows requested into the same
  // registers (in flight during the softmax, the second product and the stores),
  // then the rest.
  auto step = [&](int tile, Tile& T) {
    // the operands are read from LDS per tile, not held in registers across
    // tiles (the loop writes no LDS, so nothing else stops them being hoisted)
    asm volatile("" ::: "memory");
    f32x16_t sacc[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      sacc[x] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) sacc[x] = mfma32x32(sm.kop[x][s][lane], T.q[s], sacc[x]);
    }
    const int code = T.code, t = T.t;
    fetch(tile + 4, T);
    // keys past a row's position exist only when the block holds the row's own
    // position: mask only then (the same branch for the whole wave)
    const bool masked = __any(t < last_key);
    const int rel = t - key0;  // compared with constant key offsets
    if (masked) {  // exp2 of -inf is 0, since c > 0
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * x + 8 * (j >> 2) + (j & 3) > rel) sacc[x][j] = -INFINITY;
    }
    float mr = sacc[0][0];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int j = 0; j < 16; ++j) mr = fmaxf(mr, sacc[x][j]);
    mr = pair_max(mr);  // finite: the block's first key is visible
    const float mc = mr * c;
    float lsum = 0.f;  // the normaliser sums the fp32 probabilities
    uint4 pb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = fast_exp2(fmaf(sacc[m >> 1][8 * (m & 1) + u], c, -mc));
      if constexpr (CIS) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const float4 w = *reinterpret_cast<const float4*>(&sm.cisw[16 * m + 8 * a + 4 * g]);
          p[4 * a] *= w.x; p[4 * a + 1] *= w.y; p[4 * a + 2] *= w.z; p[4 * a + 3] *= w.w;
        }
      }
      lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pb[m] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    }
    lsum = pair_sum(lsum);
    f32x16_t acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      acc[n] = f32x16_t{};
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[n] = mfma32x32(sm.vop[n][m][lane], pb[m], acc[n]);
    }
    const uint32_t slot = uint32_t(code >> 6) * uint32_t(k_sel) + uint32_t(code & 63);
    char* pp = pbase + (slot * uint32_t(heads * D * 2) + p_lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x16_t& a = acc[i >> 1];
      const int j = 8 * (i & 1);
      stream_store(reinterpret_cast<bf16_t*>(pp + i * 32 * G),
                   make_uint4(pack2(a[j], a[j + 1]), pack2(a[j + 2], a[j + 3]),
                              pack2(a[j + 4], a[j + 5]), pack2(a[j + 6], a[j + 7])));
    }
    // lane half 0 stores the maximum, half 1 the sum
    stream_store(reinterpret_cast<float*>(mbase + (slot * uint32_t(heads * 8) + m_lane)), g ? lsum : mc);
  };

  Tile T;
  fetch(wave, T);
  for (int tile = wave; tile < n_tiles; tile += 4) step(tile, T);
}

// Grid: one dimension over groups of 16 query vectors (row * heads + head);
// 16 threads per query vector, 8 dims each.  A place is valid when its id is
// >= 0, its block starts at or before the row's position and no earlier place
// of the row holds the same id (the partial kernel writes the first such
// place only).
__global__ __launch_bounds__(256) void block_merge_kernel(
    const bf16_t* __restrict__ po, const float2* __restrict__ pml, const int* __restrict__ indices,
    int k_sel, const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int heads,
    int kv_heads, long n_qv, bf16_t* __restrict__ out, float* __restrict__ out_f32,
    float* __restrict__ lse) {
  const int tid = threadIdx.x, sub = tid & 15, lane = tid & 63;
  const long qv = long(blockIdx.x) * 16 + (tid >> 4);
  const bool in = qv < n_qv;
  const long qc = in ? qv : n_qv - 1;
  const int row = int(qc / heads), head = int(qc % heads);
  const int kv = head / (heads / kv_heads);
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int t = (row - cu_q[lo]) + ((cu_k[lo + 1] - cu_k[lo]) - (cu_q[lo + 1] - cu_q[lo]));
  const int* ids = indices + (size_t(row) * kv_heads + kv) * k_sel;

  const int grp = lane & 48;
  const int rounds = (k_sel + 15) >> 4;
  const unsigned long long valid = valid_places(ids, k_sel, t, sub, grp);

  // weights: lane `sub` of the group takes places sub, sub + 16, ...: their
  // (max, sum), the group's maximum M, its weight exp2(max - M) (0 for an
  // invalid place) into LDS, and the normaliser L = sum of weight * sum
  __shared__ float wsm[16][kMaxPlaces];
  const int g = tid >> 4;
  // (max, sum) of place p at (row * k_sel + p) * heads + head; its dims 8 sub ..
  // at pbase + p * heads * 128 (the region layout of the partial kernel)
  const int G = heads / kv_heads, hg = head % G;
  const size_t base = size_t(row) * k_sel * heads + head;
  const size_t pbase = (size_t(row) * k_sel * heads + size_t(kv) * G) * kHeadDim +
                       (sub >> 1) * (16 * G) + 16 * hg + 8 * (sub & 1);
  float mj[kMaxPlaces / 16], lj[kMaxPlaces / 16];
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMaxPlaces / 16; ++u) {
    const int p = 16 * u + sub;
    const bool ok = u < rounds && ((valid >> p) & 1ull);
    const float2 ml = ok ? pml[base + size_t(p) * heads] : make_float2(-INFINITY, 0.f);
    mj[u] = ml.x;
    lj[u] = ml.y;
    M = fmaxf(M, ml.x);
  }
#pragma unroll
  for (int x = 8; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
  float Ls = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxPlaces / 16; ++u) {
    if (u >= rounds) break;
    const float w = mj[u] == -INFINITY ? 0.f : fast_exp2(mj[u] - M);
    Ls += w * lj[u];
    wsm[g][16 * u + sub] = w;
  }
#pragma unroll
  for (int x = 8; x >= 1; x >>= 1) Ls += __shfl_xor(Ls, x);
  __builtin_amdgcn_wave_barrier();  // the group's lanes are in one wave; LDS keeps its order

  // the weighted sum of the partial outputs, every load of a batch in flight together
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < k_sel; p0 += kMergeBatch) {
    float w[kMergeBatch];
    uint4 x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int p = p0 + u;
      w[u] = p < k_sel ? wsm[g][p] : 0.f;
      x[u] = w[u] != 0.f ? stream_load(po + pbase + size_t(p) * heads * kHeadDim)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      float f[8];
      f[0] = bf16lo(x[u].x); f[1] = bf16hi(x[u].x); f[2] = bf16lo(x[u].y); f[3] = bf16hi(x[u].y);
      f[4] = bf16lo(x[u].z); f[5] = bf16hi(x[u].z); f[6] = bf16lo(x[u].w); f[7] = bf16hi(x[u].w);
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] += w[u] * f[d];
    }
  }
  if (!in) return;
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  if (out_f32 != nullptr) {
    float* dst = out_f32 + size_t(qv) * kHeadDim + 8 * sub;
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  } else {
    *reinterpret_cast<uint4*>(out + size_t(qv) * kHeadDim + 8 * sub) =
        make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                   pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
  }
  if (lse != nullptr && sub == 0) lse[qv] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
}

// ------------------------------------------------ gradient dq, key-block stationary
//
// The dq of the selected attention (the exact gradient of the forward without
// CIS, for a given upstream gradient dO; the forward's natural-log normaliser
// lse and delta = dO . O given): per (row, head) over the row's keys J,
// p = exp(scale q.k - lse), ds = p (dO.v - delta), dq = scale sum_J ds k.  As
// in the forward, one workgroup per (sequence, KV head, 1024-row chunk, 64-key
// block) walks the rows that list the block in tiles of 16 query vectors;
// per tile S^T = K Q^T and dP^T = V dO^T (16 MFMAs each), then
// dq^T += K^T dS^T (16 MFMAs, dS^T packed straight into the B operand), and the
// block's share of dq (without the scale) goes out as bf16 at (row, place,
// head).  block_dq_sum_kernel adds the valid places of every (row, head).

struct DqLds {
  // 16x16x32 bf16 operands in lane order (A: lane l holds row l % 16 at k
  // indices 8 (l / 16) .. +7; the accumulator: column l % 16, rows 4 (l / 16) + e)
  uint4 kop[16][64];   // A of S^T = K Q^T: [4 s + kk][lane] = key 16 s + c16, dims 32 kk + 8 r4 ..
  uint4 vop[16][64];   // A of dP^T = V dO^T: V rows in the layout of kop
  uint4 ktop[16][64];  // A of dq^T += K^T dS^T: [8 h + n][lane] = dim 8 c16 + n, keys 32 h + 16 (u / 4) + 4 r4 + u % 4
  bf16_t stage[4][16 * kLdsRow];
  uint16_t list[kScanRows];
  int n_list;
};

template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void block_dq_partial_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ indices, int k_sel,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int kv_heads, int nb_max,
    int n_chunk, float scale_log2, bf16_t* __restrict__ pq) {
  constexpr int E = 16 / G;
  constexpr int D = kHeadDim;
  __shared__ DqLds sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const BlockUnit U = block_unit(cu_q, cu_k, kv_heads, nb_max, n_chunk);
  const int blk = U.blk, kv = U.kv, kstart = U.kstart, L = U.L, q0 = U.q0, off = U.off;
  const int r_lo = U.r_lo, r_hi = U.r_hi, r_first = U.r_first;
  if (r_first >= r_hi || kBlock * blk >= L) return;  // the same for the whole workgroup
  const int heads = kv_heads * G;

  // operands straight from K and V (rows past the sequence end repeat its last
  // row; masked), requested before the index scan: wave w loads K and V slice w
  // (kop, vop) and the eight K rows of half w / 2 for K^T outputs tiles
  // 4 (w % 2) .. +3 (ktop)
  if (tid == 0) sm.n_list = 0;
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = k + size_t(kstart) * rs + size_t(kv) * D;
  const bf16_t* vb = v + size_t(kstart) * rs + size_t(kv) * D;
  uint4 lk[4], lv[4], lt[8];
  {
    const size_t kr = size_t(min(kBlock * blk + 16 * wave + c16, L - 1)) * rs;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      lk[kk] = ld16(kb + kr + 32 * kk + 8 * r4);
      lv[kk] = ld16(vb + kr + 32 * kk + 8 * r4);
    }
    const int h = wave >> 1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = 32 * h + 16 * (u >> 2) + 4 * r4 + (u & 3);
      lt[u] = ld16(kb + size_t(min(kBlock * blk + key, L - 1)) * rs + 8 * c16);
    }
  }
  __syncthreads();  // n_list = 0 seen by every wave
  scan_rows(sm, indices, k_sel, kv_heads, kv, q0, r_lo, r_first, r_hi, blk);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    sm.kop[4 * wave + kk][lane] = lk[kk];
    sm.vop[4 * wave + kk][lane] = lv[kk];
  }
  {
    const int h = wave >> 1, n0 = 4 * (wave & 1);
#pragma unroll
    for (int n = n0; n < n0 + 4; ++n) {
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t a = (&lt[2 * x].x)[n >> 1], c = (&lt[2 * x + 1].x)[n >> 1];
        w[x] = (n & 1) ? (a >> 16) | (c & 0xFFFF0000u) : (a & 0xFFFFu) | (c << 16);
      }
      sm.ktop[8 * h + n][lane] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __syncthreads();
  const int n_list = sm.n_list;
  const int n_tiles = (n_list + E - 1) / E;
  if (wave >= n_tiles) return;  // no barrier below

  const int ent = c16 / G, hg = c16 % G;
  const int key0 = kBlock * blk + 4 * r4;
  const int last_key = kBlock * blk + kBlock - 1;
  bf16_t* stg = sm.stage[wave];
  struct Tile {
    int t;
    float lse2, dlt;
    uint4 q[4], d[4];
  };
  // tiles past the wave's last are clamped to the last one (no branch around the
  // prefetch); a slot past the list repeats the last entry and stores nothing
  auto fetch = [&](int tile, Tile& T) {
    tile = min(tile, n_tiles - 1);
    const int li = tile * E + ent;
    const int code = sm.list[li < n_list ? li : n_list - 1];
    T.t = off + r_lo + (code >> 6);
    const size_t hr = size_t(q0 + r_lo + (code >> 6)) * heads + kv * G + hg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      T.q[kk] = ld16(q + hr * D + 32 * kk + 8 * r4);
      T.d[kk] = ld16(dout + hr * D + 32 * kk + 8 * r4);
    }
    T.lse2 = lse[hr] * kLog2e;
    T.dlt = delta[hr];
  };
  auto compute = [&](int tile, const Tile& T) {
    f32x4_t sacc[4], dpacc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sacc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dpacc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sacc[s] = mfma32(sm.kop[4 * s + kk][lane], T.q[kk], sacc[s]);
        dpacc[s] = mfma32(sm.vop[4 * s + kk][lane], T.d[kk], dpacc[s]);
      }
    }
    const bool masked = __any(T.t < last_key);  // the row's own block: keys past t
    float ds[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(sacc[s][e], scale_log2, -T.lse2));
        ds[s][e] = p * (dpacc[s][e] - T.dlt);
      }
    if (masked) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key0 + 16 * s + e > T.t) ds[s][e] = 0.f;
    }
    f32x4_t acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 db = make_uint4(pack2(ds[2 * h][0], ds[2 * h][1]), pack2(ds[2 * h][2], ds[2 * h][3]),
                                  pack2(ds[2 * h + 1][0], ds[2 * h + 1][1]),
                                  pack2(ds[2 * h + 1][2], ds[2 * h + 1][3]));
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[n] = mfma32(sm.ktop[8 * h + n][lane], db, acc[n]);
    }
    // dq^T rows -> this wave's stage, then 16 contiguous bytes per lane out
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<uint4*>(&stg[c16 * kLdsRow + 32 * r4 + 8 * e]) =
          make_uint4(pack2(acc[0][e], acc[1][e]), pack2(acc[2][e], acc[3][e]),
                     pack2(acc[4][e], acc[5][e]), pack2(acc[6][e], acc[7][e]));
    __builtin_amdgcn_wave_barrier();  // LDS runs a wave's accesses in order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vq = 4 * i + r4;
      const int li = tile * E + vq / G;
      const uint4 x = *reinterpret_cast<const uint4*>(&stg[vq * kLdsRow + 8 * c16]);
      if (li < n_list) {
        const int code = sm.list[li];
        const size_t slot = (size_t(q0 + r_lo + (code >> 6)) * k_sel + (code & 63)) * heads + kv * G + vq % G;
        stream_store(pq + slot * D + 8 * c16, x);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  Tile A, B;
  fetch(wave, A);
  for (int tile = wave; tile < n_tiles; tile += 8) {
    fetch(tile + 4, B);
    compute(tile, A);
    if (tile + 4 >= n_tiles) break;
    fetch(tile + 8, A);
    compute(tile + 4, B);
  }
}

// dq[row, head] (+)= scale * (sum of the partial dq of the row's valid places);
// 16 threads per query vector (row * heads + head), 8 dims each.
__global__ __launch_bounds__(256) void block_dq_sum_kernel(
    const bf16_t* __restrict__ pq, const int* __restrict__ indices, int k_sel,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int heads,
    int kv_heads, long n_qv, float scale, int accumulate, float* __restrict__ dq) {
  const int tid = threadIdx.x, sub = tid & 15, lane = tid & 63;
  const long qv = long(blockIdx.x) * 16 + (tid >> 4);
  const bool in = qv < n_qv;
  const long qc = in ? qv : n_qv - 1;
  const int row = int(qc / heads), head = int(qc % heads);
  const int kv = head / (heads / kv_heads);
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int t = (row - cu_q[lo]) + ((cu_k[lo + 1] - cu_k[lo]) - (cu_q[lo + 1] - cu_q[lo]));
  const int* ids = indices + (size_t(row) * kv_heads + kv) * k_sel;
  const unsigned long long valid = valid_places(ids, k_sel, t, sub, lane & 48);
  const size_t base = size_t(row) * k_sel * heads + head;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < k_sel; p0 += kMergeBatch) {
    uint4 x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int p = p0 + u;
      const bool ok = p < k_sel && ((valid >> p) & 1ull);
      x[u] = ok ? stream_load(pq + (base + size_t(p) * heads) * kHeadDim + 8 * sub)
                : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      acc[0] += bf16lo(x[u].x); acc[1] += bf16hi(x[u].x);
      acc[2] += bf16lo(x[u].y); acc[3] += bf16hi(x[u].y);
      acc[4] += bf16lo(x[u].z); acc[5] += bf16hi(x[u].z);
      acc[6] += bf16lo(x[u].w); acc[7] += bf16hi(x[u].w);
    }
  }
  if (!in) return;
  float* dst = dq + size_t(qv) * kHeadDim + 8 * sub;
  float4 a = make_float4(scale * acc[0], scale * acc[1], scale * acc[2], scale * acc[3]);
  float4 b = make_float4(scale * acc[4], scale * acc[5], scale * acc[6], scale * acc[7]);
  if (accumulate & 1) {
    const float4 a0 = *reinterpret_cast<const float4*>(dst);
    const float4 b0 = *reinterpret_cast<const float4*>(dst + 4);
    a = make_float4(a.x + a0.x, a.y + a0.y, a.z + a0.z, a.w + a0.w);
    b = make_float4(b.x + b0.x, b.y + b0.y, b.z + b0.z, b.w + b0.w);
  }
  *reinterpret_cast<float4*>(dst) = a;
  *reinterpret_cast<float4*>(dst + 4) = b;
}

template <int G>
hipError_t launch_dq_g(const SelectedBwdArgs& a, int n_chunk, unsigned n_wg, hipStream_t s) {
  return launch_kernel(kKindBwdQ, block_dq_partial_kernel<G>, dim3(n_wg), dim3(256), s, a.q, a.k,
                       a.v, a.dout, a.lse, static_cast<const float*>(a.delta), a.indices, a.k_sel,
                       a.cu_q, a.cu_k, a.kv_heads, a.nb_max, n_chunk, a.scale * kLog2eHost,
                       a.dq_part);
}

template <int G, bool CIS>
hipError_t launch_partial_g(const void* q, const void* k, const void* v, const int* indices,
                            int k_sel, const float* cis, const int* cu_q, const int* cu_k,
                            int kv_heads, int nb_max, int n_chunk, unsigned n_wg, float sl2,
                            bf16_t* po, float2* pml, hipStream_t s) {
  return launch_kernel(kKindAttn, block_partial_kernel<G, CIS>, dim3(n_wg), dim3(256), s,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), indices, k_sel, cis, cu_q, cu_k, kv_heads,
                       nb_max, n_chunk, sl2, po, pml);
}

template <bool CIS>
hipError_t launch_partial_c(int G, const void* q, const void* k, const void* v, const int* idx,
                            int k_sel, const float* cis, const int* cu_q, const int* cu_k,
                            int kvh, int nb_max, int n_chunk, unsigned n_wg, float sl2,
                            bf16_t* po, float2* pml, hipStream_t s) {
  switch (G) {
    case 1: return launch_partial_g<1, CIS>(q, k, v, idx, k_sel, cis, cu_q, cu_k, kvh, nb_max, n_chunk, n_wg, sl2, po, pml, s);
    case 2: return launch_partial_g<2, CIS>(q, k, v, idx, k_sel, cis, cu_q, cu_k, kvh, nb_max, n_chunk, n_wg, sl2, po, pml, s);
    case 4: return launch_partial_g<4, CIS>(q, k, v, idx, k_sel, cis, cu_q, cu_k, kvh, nb_max, n_chunk, n_wg, sl2, po, pml, s);
    case 8: return launch_partial_g<8, CIS>(q, k, v, idx, k_sel, cis, cu_q, cu_k, kvh, nb_max, n_chunk, n_wg, sl2, po, pml, s);
    case 16: return launch_partial_g<16, CIS>(q, k, v, idx, k_sel, cis, cu_q, cu_k, kvh, nb_max, n_chunk, n_wg, sl2, po, pml, s);
    default: return hipErrorInvalidValue;
  }
}

size_t po_bytes(int rows_total, int heads, int k_sel) {
  return (size_t(rows_total) * heads * k_sel * kHeadDim * sizeof(uint16_t) + 255) & ~size_t(255);
}

}  // namespace

size_t block_attn_ws_bytes(int rows_total, int heads, int k_sel) {
  if (rows_total <= 0 || heads <= 0 || k_sel <= 0) return 0;
  return po_bytes(rows_total, heads, k_sel) +
         ((size_t(rows_total) * heads * k_sel * sizeof(float2) + 255) & ~size_t(255));
}

bool block_attn_grid_fits(int batch, int rows_total, int heads, int kv_heads, int max_seqlen_k,
                          int k_sel) {
  const long long nb = (max_seqlen_k + kBlock - 1) / kBlock;
  const long long nc = (max_seqlen_k + kScanRows - 1) / kScanRows;
  // every grid dimension holds fewer than 2^32 work-items, and the partial
  // states of one row chunk span fewer than 2^32 bytes (32-bit offsets)
  return (long long)batch * kv_heads * nb * nc * 256 <= UINT_MAX &&
         (long long)rows_total * heads * 16 <= UINT_MAX &&
         (long long)kScanRows * k_sel * heads * kHeadDim * 2 <= UINT_MAX;
}

hipError_t launch_block_attn(const void* q, const void* k, const void* v, const int* indices,
                             int k_sel, const float* cis, void* out, float* out_f32, float* lse,
                             const int* cu_q, const int* cu_k, int batch, int rows_total,
                             int heads, int kv_heads, int max_seqlen_k, float scale_log2,
                             void* ws, hipStream_t s) {
  if (rows_total == 0 || batch == 0 || max_seqlen_k == 0) return hipSuccess;
  if (k_sel > kMaxPlaces || !(scale_log2 > 0.f) ||
      !block_attn_grid_fits(batch, rows_total, heads, kv_heads, max_seqlen_k, k_sel))
    return hipErrorInvalidValue;
  const int G = heads / kv_heads;
  const int nb_max = (max_seqlen_k + kBlock - 1) / kBlock;
  const int n_chunk = (max_seqlen_k + kScanRows - 1) / kScanRows;
  const unsigned n_wg = unsigned(batch) * kv_heads * n_chunk * nb_max;
  bf16_t* po = static_cast<bf16_t*>(ws);
  float2* pml = reinterpret_cast<float2*>(static_cast<char*>(ws) + po_bytes(rows_total, heads, k_sel));
  hipError_t e = cis != nullptr
                     ? launch_partial_c<true>(G, q, k, v, indices, k_sel, cis, cu_q, cu_k, kv_heads, nb_max, n_chunk, n_wg, scale_log2, po, pml, s)
                     : launch_partial_c<false>(G, q, k, v, indices, k_sel, cis, cu_q, cu_k, kv_heads, nb_max, n_chunk, n_wg, scale_log2, po, pml, s);
  if (e != hipSuccess) return e;
  const long n_qv = long(rows_total) * heads;
  return launch_kernel(kKindCombine, block_merge_kernel, dim3(unsigned((n_qv + 15) / 16)),
                       dim3(256), s, static_cast<const bf16_t*>(po),
                       static_cast<const float2*>(pml), indices, k_sel, cu_q, cu_k, batch, heads,
                       kv_heads, n_qv, static_cast<bf16_t*>(out), out_f32, lse);
}

size_t block_dq_ws_bytes(int rows_total, int heads, int k_sel) {
  if (rows_total <= 0 || heads <= 0 || k_sel <= 0) return 0;
  return po_bytes(rows_total, heads, k_sel);
}

hipError_t launch_block_dq(const SelectedBwdArgs& a, hipStream_t s) {
  if (a.rows_total == 0 || a.batch == 0 || a.max_seqlen_k == 0) return hipSuccess;
  if (a.k_sel > kMaxPlaces ||
      !block_attn_grid_fits(a.batch, a.rows_total, a.heads, a.kv_heads, a.max_seqlen_k, a.k_sel))
    return hipErrorInvalidValue;
  const int G = a.heads / a.kv_heads;
  const int n_chunk = (a.max_seqlen_k + kScanRows - 1) / kScanRows;
  const unsigned n_wg = unsigned(a.batch) * a.kv_heads * n_chunk * a.nb_max;
  hipError_t e;
  switch (G) {
    case 1: e = launch_dq_g<1>(a, n_chunk, n_wg, s); break;
    case 2: e = launch_dq_g<2>(a, n_chunk, n_wg, s); break;
    case 4: e = launch_dq_g<4>(a, n_chunk, n_wg, s); break;
    case 8: e = launch_dq_g<8>(a, n_chunk, n_wg, s); break;
    case 16: e = launch_dq_g<16>(a, n_chunk, n_wg, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const long n_qv = long(a.rows_total) * a.heads;
  return launch_kernel(kKindBwdQMerge, block_dq_sum_kernel, dim3(unsigned((n_qv + 15) / 16)),
                       dim3(256), s, static_cast<const bf16_t*>(a.dq_part), a.indices, a.k_sel,
                       a.cu_q, a.cu_k, a.batch, a.heads, a.kv_heads, n_qv, a.scale, a.accumulate,
                       a.dq);
}

}  // namespace nsa
