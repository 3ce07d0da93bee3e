// Attention backward on the matrix cores (bf16 operands, fp32 accumulation).
//
// What is computed is what backward.hip computes (the exact gradient of each
// prefill branch; DeepSeek NSA with Triton, introduction and section 2.3, and
// section 1.1 for the branches): per (row, query head h of KV group g) over the
// row's keys J, with p = exp(scale q.k - lse) from the forward's normaliser,
//   dV_J += p dO^T,  ds = p * (V_J dO - delta),  delta = dO . O,
//   dq = scale ds K_J,  dK_J += scale ds q^T.
// The contractions are dense 16 x 16 tiles once the work is arranged by tiles of
// 16 "query vectors" (a query vector is one (row, head) pair of a group: 16/G
// rows of G heads) against 16 keys:
//
// bwd_dkdv_mfma_kernel -- key-block stationary.  A workgroup holds one 64-key
//   block of one (sequence, KV head) (wave w: keys 16w .. 16w+15, its K and V
//   rows in registers as MFMA B operands) and walks the query tiles that see the
//   block (a row list for the selected branch, one contiguous range of
//   positions for the window and compressed branches).  Each tile's q and dO
//   rows are staged in LDS once for the four waves.
//   Per tile and wave: S = Q K^T and dP = dO V^T on four v_mfma_f32_16x16x32_bf16
//   each; their accumulators hold (query 4r4+e, key c16), which is exactly half
//   of a B operand of the tiles dV^T += dO^T P and dK^T += Q^T dS (contraction
//   over query vectors), so P and dS go to the matrix cores as packed
//   registers.  Tiles are taken two at a time, so those products run on
//   16x16x32 tiles over both tiles' 32 query vectors (the 16x16x16 form does
//   half the work per instruction); dO^T and Q^T are read from the staged rows
//   with gfx950's transposing LDS read (ds_read_b64_tr_b16).
// bwd_dq_mfma_kernel -- query-tile stationary (window and compressed branches).
//   A workgroup holds eight query tiles for the compressed branch (two per
//   wave, so each operand read from LDS feeds two products; four for the
//   window; consecutive rows, which see nearly the same keys) with Q and dO in
//   registers as B operands, and
//   walks the 64-key blocks they see, each staged in LDS once for the four
//   waves (K rows, V rows).  Per 16-key slice: S^T = K Q^T and
//   dP^T = V dO^T (accumulators (key 4r4+e, query c16)); per two slices
//   dQ^T += K^T dS^T on 16x16x32 tiles, with dS^T packed straight into the B
//   operand and K^T read transposed from the K rows.
// bwd_dq_sel_mfma_kernel -- dq of the selected branch, one (row, KV head) per
//   workgroup: the G heads are the tile's columns (columns past G masked), each
//   listed block is staged in LDS once (K rows), wave w takes its keys
//   16w .. 16w+15 (V rows straight into registers), and the four waves' dq^T
//   are summed through LDS at the end.  K^T operands come from the staged rows
//   through the transposing read.
// Masked keys (outside the row's key set, or past the sequence) get p = 0.
#include <algorithm>

#include "bwd_keys.h"
#include "common.h"
#include "launch.h"

namespace nsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// Rows of a key block's list one dk/dv workgroup takes: the chunks of one block
// add their sums with fp32 atomics, so the compressed branch, whose blocks are
// seen by nearly every later row, takes longer chunks (fewer atomics); 1024
// elsewhere (selected: 256 and 2048 measured slower; a window block's rows,
// 64 + window - 1, then fit one chunk for windows up to 961).
constexpr int rows_per_chunk(int mode) { return mode == kBwdCompressed ? 2048 : 1024; }

// Unpadded 256-byte rows whose sixteen 16-byte chunks are XOR-swizzled by
// swz(row) = 2 (row % 8) + (row / 8) % 2.  The transposing reads below
// (16 lanes: 4 rows x 32 contiguous bytes) and the staging writes are then
// conflict-free, and so are the row reads of the 16x16x32 operands (16 rows,
// one chunk each) in the chunk order kslot gives.  tile_at: the element
// offset of logical chunk c of a row.
__device__ __forceinline__ int swz(int row) { return 2 * (row & 7) + ((row >> 3) & 1); }
__device__ __forceinline__ int tile_at(int row, int c) { return row * kHeadDim + 8 * (c ^ swz(row)); }

// The dims a lane feeds to MFMA step i of a 128-dim contraction (16x16x32:
// lane row r4 supplies k-slots 8 r4 .. 8 r4 + 7): the 16-byte chunk
// 4 i + kslot(r4), the two bits of r4 swapped.  Both operands of a product
// take the same chunk, so the sum is unchanged; with the swizzle above this
// order keeps the staged-row reads (16 rows, one chunk each) off each other's
// banks, which the plain order 4 i + r4 does not on gfx950 (two passes per
// read, measured with bank-conflict counters over the access pattern alone).
__device__ __forceinline__ int kslot(int r4) { return ((r4 & 1) << 1) | (r4 >> 1); }

// The 16x16x16 A operand of X^T for dims 16 n .. 16 n + 15 and rows r0 .. r0 + 15
// of a swizzled row tile X (query vectors or keys): lane (c16, r4) gets
// X[r0 + 4 r4 + j][16 n + c16], j = 0..3, through one ds_read_b64_tr_b16.
// Within 16 lanes that read hands lane i, as its element j, element i % 4 of
// the 8 bytes at the address of lane 4 j + i / 4; so lane k addresses row
// r0 + 4 r4 + k / 4 at dims 16 n + 4 (k % 4).
typedef short s16x4_t_ __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr(const bf16_t* tile, int r0, int n) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, r4 = lane >> 4;
  const int row = r0 + 4 * r4 + (c16 >> 2);
  const int d = 16 * n + 4 * (c16 & 3);
  const bf16_t* p = tile + tile_at(row, d >> 3) + (d & 7);
  const s16x4_t_ x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t_*)(p));
  return __builtin_bit_cast(uint2, x);
}

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
// the 8 bf16 of a 16x16x32 operand from two 4-element halves: k slots
// 8 r4 .. 8 r4 + 3 from a, 8 r4 + 4 .. 8 r4 + 7 from b
__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ uint2 pack4(const float x[4]) {
  const bf16x2_t lo = {(__bf16)x[0], (__bf16)x[1]};
  const bf16x2_t hi = {(__bf16)x[2], (__bf16)x[3]};
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// One query tile (16 query vectors) staged by direct-to-LDS loads
// (global_load_lds: lane i of a wave writes its 16 (or 4) bytes at the wave's
// LDS base + 16 i (4 i)): q and dO rows as swizzled rows (each lane loads the
// logical chunk that lands at its place; the transposed operands are read
// from them with read_tr), and the natural-log normalisers and deltas of the
// 16 query vectors (lanes 16..63 repeat them).  A ring of pairs of slots keeps
// all but one pair in flight without holding them in registers.
struct QSlot {
  bf16_t q[16 * kHeadDim];
  bf16_t d[16 * kHeadDim];
  float lse[kWave];
  float delta[kWave];
};
// two tiles consumed per step (their dV, dK products share 16x16x32 tiles)
struct QPair {
  QSlot t[2];
};
// pairs in the ring: three (52 KB), two for the selected branch (its staged
// row list would push three workgroups' rings past a CU's 160 KB of LDS)
constexpr int q_pairs(int mode) { return mode == kBwdSelected ? 2 : 3; }

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void lds_load16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 4, 0, 0);
}
// Wait until at most N of this wave's vector-memory loads are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, the other counters
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Runs f on the given LDS regions declared non-aliasing, so the compiler does
// not order the reads of one (the current slot, the row list) behind the loads
// still in flight into another (the loop's explicit waits order them against
// earlier loads).  Every LDS read in the ring's loop goes through one of these.
template <typename A, typename B, typename F>
__device__ __forceinline__ void with_noalias(A* __restrict__ a, B* __restrict__ b, F&& f) {
  f(a, b);
}
template <typename A, typename B, typename C, typename F>
__device__ __forceinline__ void with_noalias(A* __restrict__ a, B* __restrict__ b, C* __restrict__ c,
                                             F&& f) {
  f(a, b, c);
}


// dK, dV of one (sequence, KV head, 64-key block) over one chunk of the rows
// that see it.  Grid: (slot, chunk).
template <int G, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_dkdv_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ cnt, const int* __restrict__ off,
    const int2* __restrict__ list, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    const int* __restrict__ cu_kv, int window, int accumulate, int heads, int kv_heads,
    int nb_max, int n_bg, int n_chunk, float scale_log2, float scale, float* __restrict__ dk,
    float* __restrict__ dv) {
  constexpr int kRowsPerTile = 16 / G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  int slot, chunk;
  if constexpr (MODE != kBwdCompressed) {
    slot = blockIdx.x;
    chunk = blockIdx.y;
  } else {
    // One-dimensional grid over groups (chunk, sequence, KV head) of nb_max key
    // blocks.  Workgroups go to the 8 XCDs in launch order modulo 8; group q
    // runs on XCD q % 8, which takes its groups in turn, so the key blocks that
    // read one chunk's rows share that XCD's L2, and the groups of later,
    // longer chunks spread over all XCDs.  Groups past the last (the count
    // rounded up to 8) are empty.  (The window branch has too few groups, two
    // chunks of very different lengths per sequence and KV head, to balance
    // the XCDs this way.)
    const int j = int(blockIdx.x) >> 3;
    const int grp = (int(blockIdx.x) & 7) + 8 * (j / nb_max);
    if (grp >= n_bg * n_chunk) return;  // uniform
    chunk = grp / n_bg;
    slot = j % nb_max + nb_max * (grp % n_bg);
  }
  const int id = slot % nb_max;
  const int g = (slot / nb_max) % kv_heads;
  const int b = slot / (nb_max * kv_heads);
  const int kstart = cu_kv[b], len = cu_kv[b + 1] - kstart;
  if (kBlock * id >= len) return;  // uniform: no key of this sequence here
  int n, t_lo = 0, row_lo = 0;
  if constexpr (MODE == kBwdSelected) n = cnt[slot];
  else n = implicit_rows<MODE>(b, id, len, window, cu_q, cu_k, t_lo, row_lo);
  constexpr int kRowsPerChunk = rows_per_chunk(MODE);
  const int e_begin = chunk * kRowsPerChunk;
  if (chunk > 0 && e_begin >= n) return;   // uniform: no rows left for this chunk
  if (n == 0 && (accumulate & 2)) return;  // nothing to add
  const int e_end = min(n, e_begin + kRowsPerChunk);
  const int first = MODE == kBwdSelected ? off[slot] : 0;


  // this wave's 16 keys as B operands: key c16 of the slice, dims 32i + 8 r4 .. +8
  const size_t rs = size_t(kv_heads) * kHeadDim;
  const int key = kBlock * id + 16 * wave + c16;
  const bool key_ok = key < len;
  const bf16_t* krow = k + (size_t(kstart + min(key, len - 1))) * rs + size_t(g) * kHeadDim;
  const bf16_t* vrow = v + (size_t(kstart + min(key, len - 1))) * rs + size_t(g) * kHeadDim;
  uint4 kb[4], vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kb[i] = ld16(krow + 32 * i + 8 * kslot(r4));
    vb[i] = ld16(vrow + 32 * i + 8 * kslot(r4));
  }
  f32x4_t acck[8], accv[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    acck[dt] = {0.f, 0.f, 0.f, 0.f};
    accv[dt] = {0.f, 0.f, 0.f, 0.f};
  }

  // One query tile against the wave's 16 keys: S = Q K^T and dP = dO V^T, and
  // from them P and dS packed as B operands (query 4 r4 + e, key c16).  sl the
  // staged tile (q and dO rows, the natural-log normalisers and deltas of its
  // 16 query vectors), tpos(qv) the position of query vector qv (-1: none).
  auto scores = [&](const QSlot* sl, auto&& tpos, uint2& pb, uint2& dsb) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = mfma32(*reinterpret_cast<const uint4*>(&sl->q[tile_at(c16, 4 * i + kslot(r4))]), kb[i], s);
      dp = mfma32(*reinterpret_cast<const uint4*>(&sl->d[tile_at(c16, 4 * i + kslot(r4))]), vb[i], dp);
    }
    // the lane's four query vectors 4 r4 .. 4 r4 + 3: one 16-byte read each
    const float4 l4 = *reinterpret_cast<const float4*>(sl->lse + 4 * r4);
    const float4 d4 = *reinterpret_cast<const float4*>(sl->delta + 4 * r4);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
    float p[4], ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tq_ = tpos(4 * r4 + e);
      const bool ok = key_ok && tq_ >= 0 && key_visible<MODE>(key, tq_, len, window);
      // masked keys take exp2(-inf) = 0 (no branch around the exponential)
      p[e] = fast_exp2(ok ? fmaf(s[e], scale, -lv[e]) * kLog2e : -INFINITY);
      ds[e] = p[e] * (dp[e] - dv4[e]);
    }
    pb = pack4(p);
    dsb = pack4(ds);
  };
  // Two query tiles x, y: dV^T += dO^T P and dK^T += Q^T dS over their 32 query
  // vectors on 16x16x32 tiles; k slots 8 r4 + j hold query vector 4 r4 + j of x
  // (j < 4) and 4 r4 + j - 4 of y (j >= 4) in both operands, dO^T and Q^T read
  // from the staged rows with the transposing read.
  auto compute2 = [&](const QSlot* x, const QSlot* y, auto&& tpos_x, auto&& tpos_y) {
    uint2 px, dsx, py, dsy;
    scores(x, tpos_x, px, dsx);
    scores(y, tpos_y, py, dsy);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      accv[dt] = mfma32(cat(read_tr(x->d, 0, dt), read_tr(y->d, 0, dt)), cat(px, py), accv[dt]);
      acck[dt] = mfma32(cat(read_tr(x->q, 0, dt), read_tr(y->q, 0, dt)), cat(dsx, dsy), acck[dt]);
    }
  };
  const int n_tiles = (e_end - e_begin + kRowsPerTile - 1) / kRowsPerTile;

  const int n_pairs = (n_tiles + 1) / 2;
  constexpr int kQPairs = q_pairs(MODE);

  // Query tiles go straight from memory into a ring of LDS slots, taken two at a
  // time (a pair), kQPairs - 1 pairs in flight.  Every wave issues 2 loads per
  // tile (waves 0 and 1 one more, for the scalars), also for the tiles past the
  // last (they repeat it into a slot whose query vectors are all masked, or
  // that no one reads), so the count of loads issued after a pair's is fixed
  // and the waits are exact.  The selected branch's rows come from the block's
  // list: the chunk's entries are loaded into LDS first, so no tile's
  // addresses wait on a load still in the ring's queue.
  // (Plain loads and LDS writes: a load into LDS outside the ring would make
  // the compiler order every later LDS read behind the ring's loads.)
  constexpr int kListChunk = MODE == kBwdSelected ? kRowsPerChunk : 1;
  __shared__ int2 ents[kListChunk];
  if constexpr (MODE == kBwdSelected) {
#pragma unroll
    for (int u = 0; u < kListChunk / kThreads; ++u) {
      const int e = e_begin + kThreads * u + tid;
      if (e < e_end) ents[kThreads * u + tid] = list[first + e];
    }
    __syncthreads();
  }
  // row and position of entry e of the chunk (ent: the staged list)
  auto row_at = [&](const int2* ent, int e) {
    if constexpr (MODE == kBwdSelected) return ent[e - e_begin];
    else return make_int2(row_lo + e, t_lo + e);
  };
  __shared__ QPair ring[kQPairs];
  auto issue = [&](const int2* ent, int tile, QSlot* slot) {
    const int e0 = e_begin + min(tile, n_tiles - 1) * kRowsPerTile;
    const int v = 4 * wave + (lane >> 4);  // the query vector whose row part this lane loads
    const int2 rt = row_at(ent, min(e0 + v / G, e_end - 1));
    const size_t hrow = size_t(rt.x) * heads + size_t(g) * G + (v % G);
    const size_t src = hrow * kHeadDim + 8 * ((lane & 15) ^ swz(v));
    lds_load16(q + src, slot->q + 4 * kHeadDim * wave);
    lds_load16(dout + src, slot->d + 4 * kHeadDim * wave);
    if (wave < 2) {
      const int qv = lane & 15;
      const int2 rs_ = row_at(ent, min(e0 + qv / G, e_end - 1));
      const size_t hs = size_t(rs_.x) * heads + size_t(g) * G + (qv % G);
      lds_load4(wave == 0 ? static_cast<const void*>(lse + hs) : static_cast<const void*>(delta + hs),
                wave == 0 ? static_cast<void*>(slot->lse) : static_cast<void*>(slot->delta));
    }
  };
  auto issue_pair = [&](const int2* ent, int pr, QPair* slot) {
    issue(ent, 2 * pr, &slot->t[0]);
    issue(ent, 2 * pr + 1, &slot->t[1]);
  };
  if (n_pairs > 0) {
#pragma unroll
    for (int t = 0; t < kQPairs - 1; ++t)
      with_noalias(static_cast<const int2*>(ents), &ring[t],
                   [&](const int2* ent, QPair* nxt) { issue_pair(ent, t, nxt); });
  }
  // unrolled by the ring size, so every slot's LDS offsets are constants
  for (int p0 = 0; p0 < n_pairs; p0 += kQPairs) {
#pragma unroll
    for (int r = 0; r < kQPairs; ++r) {
      const int pr = p0 + r;
      if (pr >= n_pairs) break;
      // pair pr has landed once at most the later pairs' loads are outstanding
      if (wave < 2) wait_vm<6 * (kQPairs - 2)>();
      else wait_vm<4 * (kQPairs - 2)>();
      __builtin_amdgcn_s_barrier();  // every wave's part of pair pr is in; pair pr - 1's slots are free
      with_noalias(static_cast<const QPair*>(&ring[r]), &ring[(r + kQPairs - 1) % kQPairs],
                   static_cast<const int2*>(ents), [&](const QPair* cur, QPair* nxt, const int2* ent) {
        issue_pair(ent, pr + kQPairs - 1, nxt);
        const int e0 = e_begin + 2 * pr * kRowsPerTile;
        compute2(&cur->t[0], &cur->t[1],
                 [&](int qv) {
                   const int e = e0 + qv / G;
                   return e < e_end ? row_at(ent, e).y : -1;
                 },
                 [&](int qv) {
                   const int e = e0 + kRowsPerTile + qv / G;
                   return e < e_end ? row_at(ent, e).y : -1;
                 });
      });
    }
  }
  wait_vm<0>();  // no load into LDS still in flight when the workgroup ends

  // lane (c16, r4) holds dims 16 dt + 4 r4 .. +3 of key c16 of the wave's slice
  if (!key_ok) return;
  const size_t o = (size_t(kstart + key) * kv_heads + g) * kHeadDim + 4 * r4;
  const bool single = n <= kRowsPerChunk;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    float4 kx = make_float4(scale * acck[dt][0], scale * acck[dt][1], scale * acck[dt][2],
                            scale * acck[dt][3]);
    float4 vx = make_float4(accv[dt][0], accv[dt][1], accv[dt][2], accv[dt][3]);
    float4* pk = reinterpret_cast<float4*>(dk + o + 16 * dt);
    float4* pv = reinterpret_cast<float4*>(dv + o + 16 * dt);
    if (single && !(accumulate & 2)) {
      *pk = kx;
      *pv = vx;
    } else if (single) {
      const float4 a = *pk, c = *pv;
      *pk = make_float4(a.x + kx.x, a.y + kx.y, a.z + kx.z, a.w + kx.w);
      *pv = make_float4(c.x + vx.x, c.y + vx.y, c.z + vx.z, c.w + vx.w);
    } else {
      float* fk = dk + o + 16 * dt;
      float* fv = dv + o + 16 * dt;
      atomicAdd(fk + 0, kx.x); atomicAdd(fk + 1, kx.y); atomicAdd(fk + 2, kx.z); atomicAdd(fk + 3, kx.w);
      atomicAdd(fv + 0, vx.x); atomicAdd(fv + 1, vx.y); atomicAdd(fv + 2, vx.z); atomicAdd(fv + 3, vx.w);
    }
  }
}

// One staged 64-key block for the dq kernel: K rows and V rows (swizzled rows;
// K^T is read from the K rows with read_tr).
struct KBlockLds {
  bf16_t k[64 * kHeadDim];
  bf16_t v[64 * kHeadDim];
};

// query tiles per wave of the dq kernel: two for the compressed branch (each
// operand read from LDS feeds both), one for the window (its short key ranges
// leave less to share, and one tile keeps three waves per SIMD)
constexpr int dq_tiles_per_wave(int mode) { return mode == kBwdWindow ? 1 : 2; }

// dq of 4 dq_tiles_per_wave query tiles of one (sequence, KV head); with two
// per wave each K and V operand read from LDS feeds both tiles' products:
// grid (row group, kv head, sequence); the window and compressed key sets.
template <int G, int MODE>
__global__ __launch_bounds__(kThreads) void bwd_dq_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    const int* __restrict__ cu_kv, int window, int accumulate, int heads, int kv_heads,
    float scale_log2, float scale, float* __restrict__ dq) {
  constexpr int kRowsPerTile = 16 / G;
  constexpr int kTw = dq_tiles_per_wave(MODE);  // query tiles per wave
  constexpr int kRowsPerWg = 4 * kTw * kRowsPerTile;
  __shared__ KBlockLds S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int g = blockIdx.y, b = blockIdx.z;
  const int q0 = cu_q[b], lq = cu_q[b + 1] - q0;
  const int len = cu_k[b + 1] - cu_k[b];
  const int shift = len - lq;
  const int rbase = blockIdx.x * kRowsPerWg;
  if (rbase >= lq) return;  // uniform
  const int kstart = cu_kv[b], klen = cu_kv[b + 1] - kstart;

  // this wave's query tiles u = 0, 1: column c16 = (row rbase + 16/G (2 wave + u)
  // + c16 / G, head c16 % G)
  int t[kTw];
  bool col_ok[kTw];
  size_t hrow[kTw];
  uint4 qb[kTw][4], db[kTw][4];
  float lse2[kTw], dlt[kTw];
  f32x4_t acc[kTw][8];
#pragma unroll
  for (int u = 0; u < kTw; ++u) {
    const int rr = rbase + kRowsPerTile * (kTw * wave + u) + c16 / G;
    col_ok[u] = rr < lq;
    t[u] = col_ok[u] ? rr + shift : -1;
    hrow[u] = size_t(q0 + min(rr, lq - 1)) * heads + size_t(g) * G + (c16 % G);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qb[u][i] = col_ok[u] ? ld16(q + hrow[u] * kHeadDim + 32 * i + 8 * kslot(r4)) : make_uint4(0u, 0u, 0u, 0u);
      db[u][i] = col_ok[u] ? ld16(dout + hrow[u] * kHeadDim + 32 * i + 8 * kslot(r4)) : make_uint4(0u, 0u, 0u, 0u);
    }
    lse2[u] = col_ok[u] ? lse[hrow[u]] * kLog2e : 0.f;
    dlt[u] = col_ok[u] ? delta[hrow[u]] : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[u][dt] = {0.f, 0.f, 0.f, 0.f};
  }

  // key blocks seen by the workgroup's rows
  const int t_first = rbase + shift;
  const int t_last = min(rbase + kRowsPerWg, lq) - 1 + shift;
  int blo = 0, bhi = -1;
  if constexpr (MODE == kBwdWindow) {
    blo = max(0, t_first - window + 1) / kBlock;
    bhi = min(t_last, klen - 1) / kBlock;
  } else {
    const int nvis = t_last >= kKernel - 1 ? min(klen, (t_last - (kKernel - 1)) / kStride + 1) : 0;
    bhi = (nvis + kBlock - 1) / kBlock - 1;
  }

  // staging: thread tid moves chunks c = tid + 256 u (u < 4) of K and of V:
  // key c / 16, dims 8 (c % 16) .. +7
  const size_t rs = size_t(kv_heads) * kHeadDim;
  uint4 pk[4], pv[4];
  auto fetch = [&](int blk) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kThreads * u;
      const int kk = kBlock * blk + (c >> 4);
      const size_t ro = size_t(kstart + min(kk, klen - 1)) * rs + size_t(g) * kHeadDim + 8 * (c & 15);
      pk[u] = ld16(k + ro);
      pv[u] = ld16(v + ro);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kThreads * u, kr = c >> 4, ch = c & 15;
      *reinterpret_cast<uint4*>(&S.k[tile_at(kr, ch)]) = pk[u];
      *reinterpret_cast<uint4*>(&S.v[tile_at(kr, ch)]) = pv[u];
    }
  };

  if (blo <= bhi) fetch(blo);
  for (int blk = blo; blk <= bhi; ++blk) {
    __syncthreads();  // the previous block is no longer read
    stash();
    __syncthreads();
    if (blk + 1 <= bhi) fetch(blk + 1);
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      uint2 dsb[kTw][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sl = 2 * sp + h;
        // S^T = K Q^T and dP^T = V dO^T: (key 16 sl + 4 r4 + e, query c16)
        f32x4_t st[kTw], dpt[kTw];
#pragma unroll
        for (int u = 0; u < kTw; ++u) {
          st[u] = {0.f, 0.f, 0.f, 0.f};
          dpt[u] = {0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 ka = *reinterpret_cast<const uint4*>(&S.k[tile_at(16 * sl + c16, 4 * i + kslot(r4))]);
          const uint4 va = *reinterpret_cast<const uint4*>(&S.v[tile_at(16 * sl + c16, 4 * i + kslot(r4))]);
#pragma unroll
          for (int u = 0; u < kTw; ++u) {
            st[u] = mfma32(ka, qb[u][i], st[u]);
            dpt[u] = mfma32(va, db[u][i], dpt[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < kTw; ++u) {
          float dst[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kk = kBlock * blk + 16 * sl + 4 * r4 + e;
            const bool ok = t[u] >= 0 && kk < klen && key_visible<MODE>(kk, t[u], klen, window);
            const float p = ok ? fast_exp2(st[u][e] * scale_log2 - lse2[u]) : 0.f;
            dst[e] = p * (dpt[u][e] - dlt[u]);
          }
          dsb[u][h] = pack4(dst);
        }
      }
      // dQ^T += K^T dS^T over the two slices' 32 keys on one 16x16x32 tile per
      // 16 dims: k slots 8 r4 + j hold keys 32 sp + 4 r4 + j (j < 4) and
      // 32 sp + 16 + 4 r4 + j - 4 (j >= 4) in both operands
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint4 kt = cat(read_tr(S.k, 32 * sp, dt), read_tr(S.k, 32 * sp + 16, dt));
#pragma unroll
        for (int u = 0; u < kTw; ++u) acc[u][dt] = mfma32(kt, cat(dsb[u][0], dsb[u][1]), acc[u][dt]);
      }
    }
  }
  // lane (c16, r4): dims 16 dt + 4 r4 .. +3 of query vector c16 of each tile
#pragma unroll
  for (int u = 0; u < kTw; ++u) {
    if (!col_ok[u]) continue;
    float* out = dq + hrow[u] * kHeadDim + 4 * r4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float4 x = make_float4(scale * acc[u][dt][0], scale * acc[u][dt][1], scale * acc[u][dt][2],
                             scale * acc[u][dt][3]);
      float4* po = reinterpret_cast<float4*>(out + 16 * dt);
      if (accumulate & 1) {
        const float4 a = *po;
        x = make_float4(a.x + x.x, a.y + x.y, a.z + x.z, a.w + x.w);
      }
      *po = x;
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void bwd_dq_sel_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ indices, int k_sel,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int batch, int accumulate,
    int heads, int kv_heads, float scale_log2, float scale, float* __restrict__ dq) {
  constexpr int kRedPad = kHeadDim + 4;
  __shared__ bf16_t Ks[64 * kHeadDim];  // swizzled rows
  __shared__ float red[4][16][kRedPad];
  __shared__ int ids_s[64];
  __shared__ int nv_s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int row = int(blockIdx.x / unsigned(kv_heads)), g = int(blockIdx.x % unsigned(kv_heads));
  int b, t;
  bwd_row_position(row, cu_q, cu_k, batch, b, t);
  const int kstart = cu_k[b], len = cu_k[b + 1] - kstart;
  // usable ids of the row (id >= 0, block start <= t), in list order
  if (wave == 0) {
    const int* irow = indices + (size_t(row) * kv_heads + g) * k_sel;
    int base = 0;
    for (int s0 = 0; s0 < k_sel; s0 += kWave) {
      const int id = s0 + lane < k_sel ? irow[s0 + lane] : -1;
      const bool ok = t >= 0 && t < len && id >= 0 && id * kBlock <= t;
      const unsigned long long m = __ballot(ok);
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (ok && pos < 64) ids_s[pos] = id;
      base += __popcll(m);
    }
    if (lane == 0) nv_s = min(base, 64);
  }
  const bool col_ok = c16 < G;
  const size_t hq = size_t(row) * heads + size_t(g) * G + min(c16, G - 1);
  uint4 qb[4], db[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qb[i] = col_ok ? ld16(q + hq * kHeadDim + 32 * i + 8 * kslot(r4)) : make_uint4(0u, 0u, 0u, 0u);
    db[i] = col_ok ? ld16(dout + hq * kHeadDim + 32 * i + 8 * kslot(r4)) : make_uint4(0u, 0u, 0u, 0u);
  }
  const float lse2 = col_ok ? lse[hq] * kLog2e : 0.f;
  const float dlt = col_ok ? delta[hq] : 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const int nv = nv_s;

  // block `id`: thread tid holds K chunks c = tid + 256 u (key c / 16, dims 8 (c % 16) ..),
  // and the V row of key 16 wave + c16 (dims 32 i + 8 r4 ..); keys past t are clamped
  // to t (their p is 0)
  const size_t rs = size_t(kv_heads) * kHeadDim;
  uint4 pk[4], pv[4], vc[4];
  auto fetch = [&](int id) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kThreads * u;
      const int kk = min(kBlock * id + (c >> 4), t);
      pk[u] = ld16(k + size_t(kstart + kk) * rs + size_t(g) * kHeadDim + 8 * (c & 15));
    }
    const int kv_ = min(kBlock * id + 16 * wave + c16, t);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pv[i] = ld16(v + size_t(kstart + kv_) * rs + size_t(g) * kHeadDim + 32 * i + 8 * kslot(r4));
  };
  if (nv > 0) fetch(ids_s[0]);
  for (int p = 0; p < nv; ++p) {
    const int id = ids_s[p];
    __syncthreads();  // the previous block's rows are no longer read
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kThreads * u;
      *reinterpret_cast<uint4*>(&Ks[tile_at(c >> 4, c & 15)]) = pk[u];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) vc[i] = pv[i];
    __syncthreads();
    if (p + 1 < nv) fetch(ids_s[p + 1]);
    // S^T = K Q^T, dP^T = V dO^T: (key 16 wave + 4 r4 + e, head column c16)
    f32x4_t st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st = mfma32(*reinterpret_cast<const uint4*>(&Ks[tile_at(16 * wave + c16, 4 * i + kslot(r4))]), qb[i], st);
      dpt = mfma32(vc[i], db[i], dpt);
    }
    float ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = kBlock * id + 16 * wave + 4 * r4 + e;
      const float pr = col_ok && key <= t ? fast_exp2(st[e] * scale_log2 - lse2) : 0.f;
      ds[e] = pr * (dpt[e] - dlt);
    }
    const uint2 dsb = pack4(ds);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)  // K^T[dim 16 dt + c16][keys 16 wave + 4 r4 .. +3]
      acc[dt] = mfma16(read_tr(Ks, 16 * wave, dt), dsb, acc[dt]);
  }
  // dq^T of the wave: (dim 16 dt + 4 r4 + e, head column c16); summed over the waves
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<float4*>(&red[wave][c16][16 * dt + 4 * r4]) =
        make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
  __syncthreads();
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    float x = scale * (red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d]);
    float* po = dq + (size_t(row) * heads + size_t(g) * G + h) * kHeadDim + d;
    if (accumulate & 1) x += *po;
    *po = x;
  }
}

template <int G, int MODE>
hipError_t launch_mfma_g(const SelectedBwdArgs& a, hipStream_t s) {
  const int n_slots = a.batch * a.kv_heads * a.nb_max;
  const float scale_log2 = a.scale * kLog2eHost;
  const int max_rows = MODE == kBwdWindow ? std::min(a.max_seqlen_k, kBlock + a.window - 1)
                                          : a.max_seqlen_k;
  const int n_chunk = std::max(1, (max_rows + rows_per_chunk(MODE) - 1) / rows_per_chunk(MODE));
  const int n_bg = a.batch * a.kv_heads;
  // the compressed branch: groups of nb_max workgroups, their count rounded up
  // to a multiple of 8 (one-dimensional grid)
  const size_t n_grouped = (size_t(n_bg) * n_chunk + 7) / 8 * 8 * size_t(a.nb_max);
  if (MODE == kBwdCompressed && n_grouped > size_t(0x7fffffff)) return hipErrorInvalidValue;
  const dim3 grid = MODE != kBwdCompressed ? dim3(unsigned(n_slots), unsigned(n_chunk))
                                           : dim3(unsigned(n_grouped));
  hipError_t e = launch_kernel(kKindBwdKV, bwd_dkdv_mfma_kernel<G, MODE>, grid, dim3(kThreads), s,
                               a.q, a.k, a.v, a.dout, a.lse, static_cast<const float*>(a.delta),
                               static_cast<const int*>(a.cnt), static_cast<const int*>(a.off),
                               static_cast<const int2*>(a.list), a.cu_q, a.cu_k, a.cu_kv,
                               a.window, a.accumulate, a.heads, a.kv_heads, a.nb_max, n_bg, n_chunk, scale_log2,
                               a.scale, a.dk, a.dv);
  if (e != hipSuccess) return e;
  if (MODE == kBwdSelected && a.dq_part != nullptr) return launch_block_dq(a, s);
  if (MODE == kBwdSelected)
    return launch_kernel(kKindBwdQ, bwd_dq_sel_mfma_kernel<G>,
                         dim3(unsigned(a.rows_total) * a.kv_heads), dim3(kThreads), s, a.q, a.k,
                         a.v, a.dout, a.lse, static_cast<const float*>(a.delta), a.indices,
                         a.k_sel, a.cu_q, a.cu_k, a.batch, a.accumulate, a.heads, a.kv_heads,
                         scale_log2, a.scale, a.dq);
  constexpr int kRowsPerWg = 4 * dq_tiles_per_wave(MODE) * (16 / G);
  const unsigned gx = unsigned((a.max_seqlen_k + kRowsPerWg - 1) / kRowsPerWg);
  return launch_kernel(kKindBwdQ, bwd_dq_mfma_kernel<G, MODE>,
                       dim3(std::max(1u, gx), unsigned(a.kv_heads), unsigned(a.batch)),
                       dim3(kThreads), s, a.q, a.k, a.v, a.dout, a.lse,
                       static_cast<const float*>(a.delta), a.cu_q, a.cu_k, a.cu_kv, a.window,
                       a.accumulate, a.heads, a.kv_heads, scale_log2, a.scale, a.dq);
}

template <int MODE>
hipError_t launch_mfma_mode(const SelectedBwdArgs& a, hipStream_t s) {
  switch (a.heads / a.kv_heads) {
    case 1: return launch_mfma_g<1, MODE>(a, s);
    case 2: return launch_mfma_g<2, MODE>(a, s);
    case 4: return launch_mfma_g<4, MODE>(a, s);
    case 8: return launch_mfma_g<8, MODE>(a, s);
    case 16: return launch_mfma_g<16, MODE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int mfma_bwd_rows_per_chunk(int mode) { return rows_per_chunk(mode); }

hipError_t launch_bwd_mfma(const SelectedBwdArgs& a, hipStream_t s) {
  switch (a.mode) {
    case kBwdSelected: return launch_mfma_mode<kBwdSelected>(a, s);
    case kBwdWindow: return launch_mfma_mode<kBwdWindow>(a, s);
    case kBwdCompressed: return launch_mfma_mode<kBwdCompressed>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nsa
