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
// block_list_kernel -- one workgroup per (sequence, KV head, chunk of 1024
//   query rows): the chunk's valid places grouped by block (a 16-bit code of
//   row and place per place, and per listed block its first entry), counted
//   and placed through an LDS table of the blocks.
// block_partial_kernel -- one workgroup per (sequence, KV head, chunk of 1024
//   query rows, listed block of the chunk).  It builds the block's matrix-core
//   operands once, in LDS, for 32x32x16 bf16 tiles (K in the A layout of
//   S^T = K Q^T, V^T in the A layout of O^T = V^T P^T), takes the rows that
//   list the block from the lists, and walks them in tiles of 32 query vectors
//   (a query vector is one (row, head) pair: 32/G rows of G heads), one tile per
//   wave at a time, so a tile costs its q rows in, 32
//   v_mfma_f32_32x32x16_bf16, and its partial state out: the block's
//   unnormalised output in bf16 plus (max, sum) in fp32, at the row's place.
// block_merge_kernel -- per (row, head): the partial states of the row's valid
//   places combined with the usual log-sum-exp weights.
//
// Precision is that of the row-by-row kernel: bf16 probabilities enter the
// matrix cores, fp32 sums (the normaliser sums the fp32 probabilities); each
// partial output is rounded to bf16 once more (2^-9 relative) before the
// merge.
#include <climits>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
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

constexpr int kChunkRows = 1024;       // query rows of one chunk (one list unit)
constexpr int kMaxPlaces = 64;        // index places per row (place fits 6 bits)
constexpr int kMergeBatch = 8;        // places whose loads the merge keeps in flight together

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
  uint16_t list[kChunkRows];  // the block's list entries: (row in chunk << 6) | place
};

// The rows of one (sequence, KV head, chunk of kChunkRows query rows) unit: its
// first packed query row q0 of the sequence, its rows r_lo .. r_hi - 1 of the
// sequence (at positions off + r), the number of blocks they can list (reach),
// and its entries of the block lists, base .. base + cap - 1 (k_sel per row, in
// KV-head-major order, so the units' entries never overlap).
struct ChunkRows {
  int q0, r_lo, r_hi, off, reach, cap;
  size_t base;
};
__device__ __forceinline__ bool chunk_rows(const int* __restrict__ cu_q, const int* __restrict__ cu_k,
                                           int b, int kv, int chunk, int rows_total, int k_sel,
                                           int nb_max, ChunkRows& u) {
  u.q0 = cu_q[b];
  const int lq = cu_q[b + 1] - u.q0;
  u.off = (cu_k[b + 1] - cu_k[b]) - lq;
  u.r_lo = chunk * kChunkRows;
  if (u.r_lo >= lq) return false;
  u.r_hi = min(lq, u.r_lo + kChunkRows);
  const int t_max = u.r_hi - 1 + u.off;
  u.reach = t_max >= 0 ? min(nb_max, t_max / kBlock + 1) : 0;
  u.cap = (u.r_hi - u.r_lo) * k_sel;
  u.base = (size_t(kv) * rows_total + u.q0 + u.r_lo) * k_sel;
  return true;
}

// The (sequence, KV head, row chunk, j) of a workgroup of a one-dimensional grid
// in XCD-grouped order (the blocks of one row chunk run together on one XCD and
// share its query rows in L2): the workgroup takes the chunk's j-th listed
// block.  False when there is no such block for certain (past the chunk's rows
// or past the blocks they can list).
struct BlockUnit {
  int j, kv, b, kstart, L;
  ChunkRows u;
};
__device__ __forceinline__ bool block_unit(const int* __restrict__ cu_q, const int* __restrict__ cu_k,
                                           int kv_heads, int nb_max, int n_chunk, int rows_total,
                                           int k_sel, BlockUnit& U) {
  int m = xcd_grouped_index(int(blockIdx.x), int(gridDim.x));
  U.j = m % nb_max;
  m /= nb_max;
  const int chunk = m % n_chunk;
  m /= n_chunk;
  U.kv = m % kv_heads;
  U.b = m / kv_heads;
  if (!chunk_rows(cu_q, cu_k, U.b, U.kv, chunk, rows_total, k_sel, nb_max, U.u)) return false;
  if (U.j >= min(U.u.cap, U.u.reach)) return false;
  U.kstart = cu_k[U.b];
  U.L = cu_k[U.b + 1] - U.kstart;
  return true;
}

// The j-th listed block of a unit (from its list head) and its entries:
// false when the unit lists fewer blocks.
__device__ __forceinline__ bool listed_block(const int2* __restrict__ lhead, const BlockUnit& U,
                                             int& blk, int& start, int& n) {
  const int2 h = lhead[U.u.base + U.j];
  if (h.x < 0) return false;
  blk = h.x;
  start = h.y;
  n = (U.j + 1 < U.u.cap ? lhead[U.u.base + U.j + 1].y : U.u.cap) - start;
  return true;
}

// Valid places of one index row for position t, as a bit mask: id >= 0, block
// start <= t, and no earlier place holding the same id.  Lane `sub` of a group
// of 16 lanes (the lanes of one query vector, `grp` its first lane) checks
// places sub, sub + 16, ... (its ids, -1 past k_sel: load_place_ids) and
// compares them with the earlier places through the group; every lane of the
// group gets the whole mask.
__device__ __forceinline__ void load_place_ids(const int* __restrict__ ids, int k_sel, int sub,
                                               int (&myid)[kMaxPlaces / 16]) {
#pragma unroll
  for (int u = 0; u < kMaxPlaces / 16; ++u) myid[u] = 16 * u + sub < k_sel ? ids[16 * u + sub] : -1;
}
__device__ __forceinline__ unsigned long long valid_of_ids(const int (&myid)[kMaxPlaces / 16],
                                                           int k_sel, int t, int sub, int grp) {
  const int rounds = (k_sel + 15) >> 4;
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
__device__ __forceinline__ unsigned long long valid_places(const int* __restrict__ ids, int k_sel,
                                                          int t, int sub, int grp) {
  int myid[kMaxPlaces / 16];
  load_place_ids(ids, k_sel, sub, myid);
  return valid_of_ids(myid, k_sel, t, sub, grp);
}

// ----------------------------------------------------------------- block lists
//
// block_list_kernel -- one workgroup per (sequence, KV head, chunk of kChunkRows
// query rows): the chunk's valid places (those valid_places admits, the places
// the merge combines) grouped by block, through a table of the blocks in LDS.
// In the unit's entries (ChunkRows::base ..): code[u] = (row in chunk << 6) |
// place, block after block in increasing block order; head[j] = (block, first
// u) of the chunk's j-th listed block, then (-1, number of places) from the
// last listed block up to the number of blocks the rows can list (and once
// when there is room), which ends every workgroup that reads past the list.
constexpr int kListMaxBlocks = 8192;  // blocks a sequence may have on this path (524288 tokens)

__global__ __launch_bounds__(256) void block_list_kernel(
    const int* __restrict__ indices, int k_sel, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int kv_heads, int nb_max, int rows_total,
    uint16_t* __restrict__ lcode, int2* __restrict__ lhead) {
  __shared__ int tab[kListMaxBlocks];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = tid & 15, grp = lane & 48;
  const int kv = blockIdx.y, b = blockIdx.z;
  ChunkRows u;
  if (!chunk_rows(cu_q, cu_k, b, kv, int(blockIdx.x), rows_total, k_sel, nb_max, u)) return;
  for (int i = tid; i < u.reach; i += 256) tab[i] = 0;
  __syncthreads();
  const int rounds = (k_sel + 15) >> 4;
  // every row's valid places, 16 rows a round (16 lanes a row), the index rows of
  // kRounds rounds loaded together; FILL: place them at their block's cursor,
  // else count them
  constexpr int kRounds = 8;
  auto each_place = [&](auto fill_tag) {
    constexpr bool FILL = decltype(fill_tag)::value;
    for (int r0 = u.r_lo; r0 < u.r_hi; r0 += 16 * kRounds) {
      int myid[kRounds][kMaxPlaces / 16];
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        // every lane of a group takes part in the shuffles: rows past the chunk
        // repeat its last row and count nothing
        const int r = min(r0 + 16 * i + (tid >> 4), u.r_hi - 1);
        load_place_ids(indices + (size_t(u.q0 + r) * kv_heads + kv) * k_sel, k_sel, sub, myid[i]);
      }
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        const int r_in = r0 + 16 * i + (tid >> 4);
        const int r = min(r_in, u.r_hi - 1);
        const unsigned long long valid = valid_of_ids(myid[i], k_sel, r + u.off, sub, grp);
        if (r_in >= u.r_hi) continue;
#pragma unroll
        for (int x = 0; x < kMaxPlaces / 16; ++x) {
          if (x >= rounds) break;
          const int p = 16 * x + sub;
          if (!((valid >> p) & 1ull) || myid[i][x] >= u.reach) continue;
          if constexpr (FILL)
            lcode[u.base + atomicAdd(&tab[myid[i][x]], 1)] = uint16_t(((r - u.r_lo) << 6) | p);
          else
            atomicAdd(&tab[myid[i][x]], 1);
        }
      }
    }
  };
  each_place(std::false_type{});
  __syncthreads();
  // exclusive scan of (count, listed) over the blocks, thread tid taking `per`
  // consecutive blocks; packed as listed << 17 | count (a unit has at most
  // 2^16 places and kListMaxBlocks blocks)
  const int per = (u.reach + 255) / 256;
  int packed = 0;
  for (int i = 0; i < per; ++i) {
    const int x = tid * per + i;
    if (x < u.reach) packed += (tab[x] != 0 ? 1 << 17 : 0) + tab[x];
  }
  const int incl = wave_inclusive_scan(packed);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = incl - packed;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int all = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int total = all & 0x1FFFF, listed = all >> 17;
  int c = before & 0x1FFFF, n = before >> 17;
  for (int i = 0; i < per; ++i) {
    const int x = tid * per + i;
    if (x >= u.reach) break;
    const int cnt = tab[x];
    if (cnt != 0) lhead[u.base + n++] = make_int2(x, c);
    tab[x] = c;  // the block's cursor
    c += cnt;
  }
  const int j_end = min(u.cap, max(u.reach, listed + 1));
  for (int j = listed + tid; j < j_end; j += 256) lhead[u.base + j] = make_int2(-1, total);
  __syncthreads();
  each_place(std::true_type{});
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
    const uint16_t* __restrict__ lcode, const int2* __restrict__ lhead, int k_sel,
    const float* __restrict__ cis, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    int kv_heads, int nb_max, int n_chunk, int rows_total, float scale_log2,
    bf16_t* __restrict__ po, float2* __restrict__ pml) {
  constexpr int E = 32 / G;  // list entries per tile of 32 query vectors
  constexpr int D = kHeadDim;
  __shared__ PartialLds sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, g = lane >> 5;

  BlockUnit U;  // both returns below are the same for the whole workgroup
  if (!block_unit(cu_q, cu_k, kv_heads, nb_max, n_chunk, rows_total, k_sel, U)) return;
  int blk, start, n_list;
  if (!listed_block(lhead, U, blk, start, n_list)) return;
  const int kv = U.kv, kstart = U.kstart, L = U.L, q0 = U.u.q0, off = U.u.off, r_lo = U.u.r_lo;
  const int heads = kv_heads * G;

  // The block's operands straight from K and V (rows past the sequence end
  // repeat its last row: finite data, masked below since they lie past every
  // row's position), requested together with the block's list entries.  Waves
  // 0 and 1 load K (16-byte piece x = 128 i + tid is key x / 16, dims
  // 8 (x % 16) ..); waves 2 and 3 load V, thread t = tid - 128 taking dims
  // 8 (t % 16) .. +7 of the eight keys of step t / 32, lane half (t / 16) % 2, and
  // transposing them in registers.
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
  for (int i = tid; i < n_list; i += 256) sm.list[i] = lcode[U.u.base + start + i];
  if (CIS && tid < kBlock) sm.cisw[tid] = cis[size_t(kstart + min(kBlock * blk + tid, L - 1)) * kv_heads + kv];
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
// in the forward, one workgroup per (sequence, KV head, 1024-row chunk, listed
// block) walks the rows that list the block in tiles of 32 query vectors on
// 32x32x16 tiles: per tile S^T = K Q^T and dP^T = V dO^T (16 MFMAs each, the
// operand layouts of the forward's kop for K and V), then dq^T += K^T dS^T (16
// MFMAs, K^T in the layout of the forward's vop, dS^T packed straight from the
// accumulators into the B operand), and the block's share of dq (without the
// scale) goes out as bf16 at (row, place, head), in the forward's partial
// output layout.  block_dq_sum_kernel adds the valid places of every (row,
// head).

struct DqLds {
  uint4 kop[2][8][64];   // K: A of S^T = K Q^T (PartialLds::kop layout)
  uint4 vop[2][8][64];   // V: A of dP^T = V dO^T (the same layout)
  uint4 ktop[4][4][64];  // K^T: A of dq^T += K^T dS^T (PartialLds::vop layout)
  uint16_t list[kChunkRows];
};

template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void block_dq_partial_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const uint16_t* __restrict__ lcode,
    const int2* __restrict__ lhead, int k_sel, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int kv_heads, int nb_max, int n_chunk, int rows_total,
    float scale_log2, bf16_t* __restrict__ pq) {
  constexpr int E = 32 / G;
  constexpr int D = kHeadDim;
  __shared__ DqLds sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, g = lane >> 5;
  BlockUnit U;  // both returns below are the same for the whole workgroup
  if (!block_unit(cu_q, cu_k, kv_heads, nb_max, n_chunk, rows_total, k_sel, U)) return;
  int blk, start, n_list;
  if (!listed_block(lhead, U, blk, start, n_list)) return;
  const int kv = U.kv, kstart = U.kstart, L = U.L, q0 = U.u.q0, off = U.u.off, r_lo = U.u.r_lo;
  const int heads = kv_heads * G;

  // operands straight from K and V (rows past the sequence end repeat its last
  // row; masked): waves 0 and 1 load K pieces for kop (as the forward), waves 2
  // and 3 V pieces for vop and, as the forward's V, the K pieces of ktop
  const size_t rs = size_t(kv_heads) * D;
  const bf16_t* kb = k + size_t(kstart) * rs + size_t(kv) * D;
  const bf16_t* vb = v + size_t(kstart) * rs + size_t(kv) * D;
  const int t2 = tid & 127;
  const bf16_t* src = wave < 2 ? kb : vb;
  uint4 la[8], lt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int x = 128 * i + t2;
    la[i] = ld16(src + size_t(min(kBlock * blk + (x >> 4), L - 1)) * rs + 8 * (x & 15));
  }
  if (wave >= 2) {
    const int m = t2 >> 5, gh = (t2 >> 4) & 1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = 16 * m + 8 * (u >> 2) + 4 * gh + (u & 3);
      lt[u] = ld16(kb + size_t(min(kBlock * blk + key, L - 1)) * rs + 8 * (t2 & 15));
    }
  }
  for (int i = tid; i < n_list; i += 256) sm.list[i] = lcode[U.u.base + start + i];
  {
    uint4(*dst)[8][64] = wave < 2 ? sm.kop : sm.vop;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int x = 128 * i + t2, key = x >> 4, pc = x & 15;
      dst[key >> 5][pc & 7][(key & 31) + 32 * (pc >> 3)] = la[i];
    }
  }
  if (wave >= 2) {
    const int m = t2 >> 5, gh = (t2 >> 4) & 1, db = t2 & 15;
    const int n = db >> 2, i2 = (db >> 1) & 1, gp = db & 1;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t a = (&lt[2 * x].x)[c >> 1], b2 = (&lt[2 * x + 1].x)[c >> 1];
        w[x] = (c & 1) ? (a >> 16) | (b2 & 0xFFFF0000u) : (a & 0xFFFFu) | (b2 << 16);
      }
      const int rho = 8 * (2 * i2 + (c >> 2)) + 4 * gp + (c & 3);
      sm.ktop[n][m][rho + 32 * gh] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __syncthreads();
  const int n_tiles = (n_list + E - 1) / E;
  if (wave >= n_tiles) return;  // no barrier below

  const int ent = c32 / G, hg = c32 % G;
  const int key0 = kBlock * blk + 4 * g;  // key of score j of half x: key0 + 32 x + 8 (j / 4) + j % 4
  const int last_key = kBlock * blk + kBlock - 1;
  // chunk bases (uniform) and per-lane byte offsets below them (32 bits)
  const size_t row0 = size_t(q0 + r_lo);
  const char* qbase = reinterpret_cast<const char*>(q + row0 * heads * D);
  const char* dbase = reinterpret_cast<const char*>(dout + row0 * heads * D);
  const float* lbase = lse + row0 * heads + kv * G + hg;
  const float* ebase = delta + row0 * heads + kv * G + hg;
  char* pbase = reinterpret_cast<char*>(pq + row0 * k_sel * heads * D);
  const uint32_t q_lane = uint32_t(((kv * G + hg) * D + 64 * g) * 2);
  const uint32_t p_lane = uint32_t((kv * G * D + 16 * hg + 8 * g) * 2);

  // a slot past the list repeats the last entry (same values, same addresses),
  // so the stores need no condition
  struct Tile {
    int code, t;
    float lse2, dlt;
    uint4 q[8], d[8];
  };
  auto fetch = [&](int tile, Tile& T) {
    tile = min(tile, n_tiles - 1);
    T.code = sm.list[min(tile * E + ent, n_list - 1)];
    const uint32_t rc = uint32_t(T.code >> 6);
    T.t = off + r_lo + int(rc);
    const uint32_t o = rc * uint32_t(heads * D * 2) + q_lane;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      T.q[s] = ld16(qbase + o + 16 * s);
      T.d[s] = ld16(dbase + o + 16 * s);
    }
    T.lse2 = lbase[rc * heads] * kLog2e;
    T.dlt = ebase[rc * heads];
  };
  auto step = [&](int tile, Tile& T) {
    asm volatile("" ::: "memory");  // the operands are read from LDS per tile
    f32x16_t sacc[2], dacc[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      sacc[x] = f32x16_t{};
      dacc[x] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sacc[x] = mfma32x32(sm.kop[x][s][lane], T.q[s], sacc[x]);
        dacc[x] = mfma32x32(sm.vop[x][s][lane], T.d[s], dacc[x]);
      }
    }
    const int code = T.code, t = T.t;
    const float lse2 = T.lse2, dlt = T.dlt;
    fetch(tile + 4, T);
    const bool masked = __any(t < last_key);  // the row's own block: keys past t
    const int rel = t - key0;
    uint4 db[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float ds[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = 8 * (m & 1) + u;
        const float p = fast_exp2(fmaf(sacc[m >> 1][j], scale_log2, -lse2));
        ds[u] = p * (dacc[m >> 1][j] - dlt);
      }
      if (masked) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (16 * m + 8 * (u >> 2) + (u & 3) > rel) ds[u] = 0.f;
      }
      db[m] = make_uint4(pack2(ds[0], ds[1]), pack2(ds[2], ds[3]), pack2(ds[4], ds[5]), pack2(ds[6], ds[7]));
    }
    f32x16_t acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      acc[n] = f32x16_t{};
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[n] = mfma32x32(sm.ktop[n][m][lane], db[m], acc[n]);
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
  };
  Tile T;
  fetch(wave, T);
  for (int tile = wave; tile < n_tiles; tile += 4) step(tile, T);
}

// dq[row, head] (+)= scale * (sum of the partial dq of the row's valid places);
// 16 threads per query vector (row * heads + head), 8 dims each (lane sub: dims
// 8 sub .. +7, in the partial output layout).
__global__ __launch_bounds__(256) void block_dq_sum_kernel(
    const bf16_t* __restrict__ pq, const int* __restrict__ indices, int k_sel,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int heads,
    int kv_heads, long n_qv, float scale, int accumulate, float* __restrict__ dq) {
  const int tid = threadIdx.x, sub = tid & 15, lane = tid & 63;
  const long qv = long(blockIdx.x) * 16 + (tid >> 4);
  const bool in = qv < n_qv;
  const long qc = in ? qv : n_qv - 1;
  const int row = int(qc / heads), head = int(qc % heads);
  const int G = heads / kv_heads, kv = head / G, hg = head % G;
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int t = (row - cu_q[lo]) + ((cu_k[lo + 1] - cu_k[lo]) - (cu_q[lo + 1] - cu_q[lo]));
  const int* ids = indices + (size_t(row) * kv_heads + kv) * k_sel;
  const unsigned long long valid = valid_places(ids, k_sel, t, sub, lane & 48);
  const size_t pbase = (size_t(row) * k_sel * heads + size_t(kv) * G) * kHeadDim +
                       (sub >> 1) * (16 * G) + 16 * hg + 8 * (sub & 1);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < k_sel; p0 += kMergeBatch) {
    uint4 x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int p = p0 + u;
      const bool ok = p < k_sel && ((valid >> p) & 1ull);
      x[u] = ok ? stream_load(pq + pbase + size_t(p) * heads * kHeadDim) : make_uint4(0u, 0u, 0u, 0u);
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
hipError_t launch_dq_g(const SelectedBwdArgs& a, const uint16_t* lcode, const int2* lhead,
                       int n_chunk, unsigned n_wg, hipStream_t s) {
  return launch_kernel(kKindBwdQ, block_dq_partial_kernel<G>, dim3(n_wg), dim3(256), s, a.q, a.k,
                       a.v, a.dout, a.lse, static_cast<const float*>(a.delta), lcode, lhead,
                       a.k_sel, a.cu_q, a.cu_k, a.kv_heads, a.nb_max, n_chunk, a.rows_total,
                       a.scale * kLog2eHost, a.dq_part);
}

// The launch arguments of the partial kernel.
struct PartialArgs {
  const bf16_t *q, *k, *v;
  const uint16_t* lcode;
  const int2* lhead;
  int k_sel;
  const float* cis;
  const int *cu_q, *cu_k;
  int kv_heads, nb_max, n_chunk, rows_total;
  float scale_log2;
  bf16_t* po;
  float2* pml;
};

template <int G, bool CIS>
hipError_t launch_partial_g(const PartialArgs& a, unsigned n_wg, hipStream_t s) {
  return launch_kernel(kKindAttn, block_partial_kernel<G, CIS>, dim3(n_wg), dim3(256), s, a.q,
                       a.k, a.v, a.lcode, a.lhead, a.k_sel, a.cis, a.cu_q, a.cu_k, a.kv_heads,
                       a.nb_max, a.n_chunk, a.rows_total, a.scale_log2, a.po, a.pml);
}

template <bool CIS>
hipError_t launch_partial_c(int G, const PartialArgs& a, unsigned n_wg, hipStream_t s) {
  switch (G) {
    case 1: return launch_partial_g<1, CIS>(a, n_wg, s);
    case 2: return launch_partial_g<2, CIS>(a, n_wg, s);
    case 4: return launch_partial_g<4, CIS>(a, n_wg, s);
    case 8: return launch_partial_g<8, CIS>(a, n_wg, s);
    case 16: return launch_partial_g<16, CIS>(a, n_wg, s);
    default: return hipErrorInvalidValue;
  }
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }
size_t po_bytes(int rows_total, int heads, int k_sel) {
  return round256(size_t(rows_total) * heads * k_sel * kHeadDim * sizeof(uint16_t));
}
// the block lists: codes (2 bytes) and heads (8 bytes) per (row, KV head, place)
size_t list_code_bytes(int rows_total, int kv_heads, int k_sel) {
  return round256(size_t(rows_total) * kv_heads * k_sel * sizeof(uint16_t));
}
size_t list_bytes(int rows_total, int kv_heads, int k_sel) {
  return list_code_bytes(rows_total, kv_heads, k_sel) +
         round256(size_t(rows_total) * kv_heads * k_sel * sizeof(int2));
}

// Build the block lists of every (sequence, KV head, row chunk) into `lists`.
hipError_t launch_lists(int kind, const int* indices, int k_sel, const int* cu_q, const int* cu_k,
                        int batch, int kv_heads, int nb_max, int n_chunk, int rows_total,
                        void* lists, uint16_t*& lcode, int2*& lhead, hipStream_t s) {
  lcode = static_cast<uint16_t*>(lists);
  lhead = reinterpret_cast<int2*>(static_cast<char*>(lists) + list_code_bytes(rows_total, kv_heads, k_sel));
  return launch_kernel(kind, block_list_kernel, dim3(unsigned(n_chunk), unsigned(kv_heads), unsigned(batch)),
                       dim3(256), s, indices, k_sel, cu_q, cu_k, kv_heads, nb_max, rows_total,
                       lcode, lhead);
}

}  // namespace

size_t block_attn_ws_bytes(int rows_total, int heads, int kv_heads, int k_sel) {
  if (rows_total <= 0 || heads <= 0 || kv_heads <= 0 || k_sel <= 0) return 0;
  return po_bytes(rows_total, heads, k_sel) +
         round256(size_t(rows_total) * heads * k_sel * sizeof(float2)) +
         list_bytes(rows_total, kv_heads, k_sel);
}

bool block_attn_grid_fits(int batch, int rows_total, int heads, int kv_heads, int max_seqlen_k,
                          int k_sel) {
  const long long nb = (max_seqlen_k + kBlock - 1) / kBlock;
  const long long nc = (max_seqlen_k + kChunkRows - 1) / kChunkRows;
  // every grid dimension holds fewer than 2^32 work-items, the partial states of
  // one row chunk span fewer than 2^32 bytes (32-bit offsets), and a
  // sequence's blocks fit the list kernel's table
  return (long long)batch * kv_heads * nb * nc * 256 <= UINT_MAX &&
         (long long)rows_total * heads * 16 <= UINT_MAX &&
         (long long)kChunkRows * k_sel * heads * kHeadDim * 2 <= UINT_MAX && nb <= kListMaxBlocks;
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
  const int n_chunk = (max_seqlen_k + kChunkRows - 1) / kChunkRows;
  const unsigned n_wg = unsigned(batch) * kv_heads * n_chunk * nb_max;
  char* w = static_cast<char*>(ws);
  bf16_t* po = reinterpret_cast<bf16_t*>(w);
  w += po_bytes(rows_total, heads, k_sel);
  float2* pml = reinterpret_cast<float2*>(w);
  w += round256(size_t(rows_total) * heads * k_sel * sizeof(float2));
  PartialArgs a{static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                static_cast<const bf16_t*>(v), nullptr, nullptr, k_sel, cis, cu_q, cu_k,
                kv_heads, nb_max, n_chunk, rows_total, scale_log2, po, pml};
  uint16_t* lcode;
  int2* lhead;
  hipError_t e = launch_lists(kKindBlockLists, indices, k_sel, cu_q, cu_k, batch, kv_heads, nb_max,
                              n_chunk, rows_total, w, lcode, lhead, s);
  if (e != hipSuccess) return e;
  a.lcode = lcode;
  a.lhead = lhead;
  e = cis != nullptr ? launch_partial_c<true>(G, a, n_wg, s) : launch_partial_c<false>(G, a, n_wg, s);
  if (e != hipSuccess) return e;
  const long n_qv = long(rows_total) * heads;
  return launch_kernel(kKindCombine, block_merge_kernel, dim3(unsigned((n_qv + 15) / 16)),
                       dim3(256), s, static_cast<const bf16_t*>(po),
                       static_cast<const float2*>(pml), indices, k_sel, cu_q, cu_k, batch, heads,
                       kv_heads, n_qv, static_cast<bf16_t*>(out), out_f32, lse);
}

size_t block_dq_ws_bytes(int rows_total, int heads, int kv_heads, int k_sel) {
  if (rows_total <= 0 || heads <= 0 || kv_heads <= 0 || k_sel <= 0) return 0;
  return po_bytes(rows_total, heads, k_sel) + list_bytes(rows_total, kv_heads, k_sel);
}

hipError_t launch_block_dq(const SelectedBwdArgs& a, hipStream_t s) {
  if (a.rows_total == 0 || a.batch == 0 || a.max_seqlen_k == 0) return hipSuccess;
  if (a.k_sel > kMaxPlaces ||
      !block_attn_grid_fits(a.batch, a.rows_total, a.heads, a.kv_heads, a.max_seqlen_k, a.k_sel))
    return hipErrorInvalidValue;
  const int G = a.heads / a.kv_heads;
  const int n_chunk = (a.max_seqlen_k + kChunkRows - 1) / kChunkRows;
  const unsigned n_wg = unsigned(a.batch) * a.kv_heads * n_chunk * a.nb_max;
  uint16_t* lcode;
  int2* lhead;
  hipError_t e = launch_lists(kKindBwdLists, a.indices, a.k_sel, a.cu_q, a.cu_k, a.batch,
                              a.kv_heads, a.nb_max, n_chunk, a.rows_total,
                              reinterpret_cast<char*>(a.dq_part) + po_bytes(a.rows_total, a.heads, a.k_sel),
                              lcode, lhead, s);
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: e = launch_dq_g<1>(a, lcode, lhead, n_chunk, n_wg, s); break;
    case 2: e = launch_dq_g<2>(a, lcode, lhead, n_chunk, n_wg, s); break;
    case 4: e = launch_dq_g<4>(a, lcode, lhead, n_chunk, n_wg, s); break;
    case 8: e = launch_dq_g<8>(a, lcode, lhead, n_chunk, n_wg, s); break;
    case 16: e = launch_dq_g<16>(a, lcode, lhead, n_chunk, n_wg, s); break;
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
