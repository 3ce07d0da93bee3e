// KV offload for decode: the K/V cache stays in host memory and every step
// brings to the GPU only the selected blocks that are not already resident.
//
// What is computed (NOSA-1B core components: the core idea and the decode
// stage): the whole cache is offloaded to CPU memory, the GPU keeps only what
// scoring needs, and each step moves just the few important blocks back for the
// attention.  Here the compressed keys and pooled CIS stay in device memory, so
// scoring and selection are unchanged; a device pool of `pool_slots` block
// slots per (sequence, KV head) holds the K/V of blocks fetched by earlier
// steps.  Each step:
//   1. offload_plan_kernel: per (sequence, KV head), the listed blocks already
//      in a slot are hits; every other listed block is a miss and takes the
//      next free slot: empty slots first, then slots holding a block this step
//      does not list (each class in ascending slot order; misses in list
//      order), so blocks stay resident as long as the pool has room; the
//      slot<->block tables are updated and the misses written as a copy list.
//   2. offload_fetch_kernel: one workgroup per miss copies the block's 64 K and
//      V rows of that KV head from host memory into its slot (reads over the
//      host link; rows past the sequence end are not read).
//   3. the pool attention kernel reads the K/V rows through the slot of each
//      listed block.
// A block listed in consecutive steps is therefore fetched once; blocks of the
// previous steps stay resident while their slots are not needed.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace nsa {

namespace {

// Fill with -1 (empty slot / block not resident).
__global__ __launch_bounds__(256) void fill_neg1_kernel(int* __restrict__ p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256)
    p[i] = -1;
}

constexpr int kPlanThreads = 256;
constexpr int kSlotsPerThread = kMaxPoolSlots / kPlanThreads;

// One workgroup per (sequence, KV head); listed place p is thread p (k_sel <=
// 256), slot s is owned by thread s % 256.
__global__ __launch_bounds__(kPlanThreads) void offload_plan_kernel(
    const int* __restrict__ indices, int k_sel, int* __restrict__ slot_of, int nb_cap,
    int* __restrict__ block_of, int pool_slots, int* __restrict__ slot_ids,
    int2* __restrict__ copies, int* __restrict__ n_copy, int* __restrict__ fetched) {
  __shared__ uint32_t listed[kMaxSortBlocks / 32];
  __shared__ int free_list[kMaxPoolSlots];
  __shared__ int cnt[2][kSlotsPerThread * 4];
  __shared__ int miss_cnt[4];
  const size_t unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int i = tid; i < kMaxSortBlocks / 32; i += kPlanThreads) listed[i] = 0u;
  // the listed block of this thread's place and where it is now
  const int id = tid < k_sel ? indices[unit * k_sel + tid] : -1;
  const bool valid = id >= 0 && id < nb_cap;
  int cur = valid ? slot_of[unit * nb_cap + id] : -1;
  if (cur >= pool_slots) cur = -1;  // tables never reset: treat as not resident
  int held[kSlotsPerThread];
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int s = tid + kPlanThreads * j;
    held[j] = s < pool_slots ? block_of[unit * pool_slots + s] : 0;
  }
  __syncthreads();
  if (valid) atomicOr(&listed[id >> 5], 1u << (id & 31));
  __syncthreads();
  // free slots: class 0 empty, class 1 holding an unlisted block; ranked by
  // class, then slot: ballots per (class, slab j, wave), then one scan of each
  // class's counts (lane j * 4 + wave in slot order)
  int cls[kSlotsPerThread];  // -1 not free
  int rank[kSlotsPerThread];
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int s = tid + kPlanThreads * j;
    const int h = held[j];
    const bool in_use = h >= 0 && h < nb_cap && ((listed[h >> 5] >> (h & 31)) & 1u);
    cls[j] = s >= pool_slots || in_use ? -1 : (h < 0 ? 0 : 1);
    const unsigned long long m0 = __ballot(cls[j] == 0);
    const unsigned long long m1 = __ballot(cls[j] == 1);
    rank[j] = __popcll((cls[j] == 0 ? m0 : m1) & below);
    if (lane == 0) {
      cnt[0][j * 4 + wave] = __popcll(m0);
      cnt[1][j * 4 + wave] = __popcll(m1);
    }
  }
  const bool miss = valid && cur < 0;
  {
    const unsigned long long m = __ballot(miss);
    if (lane == 0) miss_cnt[wave] = __popcll(m);
  }
  __syncthreads();
  const int c0 = lane < kSlotsPerThread * 4 ? cnt[0][lane] : 0;
  const int c1 = lane < kSlotsPerThread * 4 ? cnt[1][lane] : 0;
  const int incl0 = wave_inclusive_scan(c0);
  const int excl0 = incl0 - c0;
  const int incl1 = wave_inclusive_scan(c1);
  const int excl1 = incl1 - c1 + __builtin_amdgcn_readlane(incl0, kWave - 1);
  const int n_free = __builtin_amdgcn_readlane(incl0, kWave - 1) + __builtin_amdgcn_readlane(incl1, kWave - 1);
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int base0 = __builtin_amdgcn_readlane(excl0, j * 4 + wave);
    const int base1 = __builtin_amdgcn_readlane(excl1, j * 4 + wave);
    if (cls[j] >= 0) free_list[rank[j] + (cls[j] == 0 ? base0 : base1)] = tid + kPlanThreads * j;
  }
  int miss_before = 0, n_miss = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    miss_before += w < wave ? miss_cnt[w] : 0;
    n_miss += miss_cnt[w];
  }
  const int mrank = miss_before + __popcll(__ballot(miss) & below);
  __syncthreads();
  // free slots >= misses whenever the tables are consistent and pool_slots >=
  // k_sel (checked on the host); a miss without a slot is left unlisted
  if (miss && mrank < n_free) {
    const int s = free_list[mrank];
    const int old = block_of[unit * pool_slots + s];  // only this thread writes slot s
    if (old >= 0 && old < nb_cap) slot_of[unit * nb_cap + old] = -1;
    slot_of[unit * nb_cap + id] = s;
    block_of[unit * pool_slots + s] = id;
    copies[unit * k_sel + mrank] = make_int2(id, s);
    cur = s;
  }
  if (tid < k_sel) slot_ids[unit * k_sel + tid] = valid ? cur : -1;
  if (tid == 0) {
    n_copy[unit] = min(n_miss, n_free);
    if (fetched != nullptr) fetched[unit] = min(n_miss, n_free);
  }
}

// One workgroup per (copy-list entry, sequence x KV head): 64 rows of 256 B of
// K and of V, 64 B per thread.
__global__ __launch_bounds__(256) void offload_fetch_kernel(
    const bf16_t* __restrict__ k_src, const bf16_t* __restrict__ v_src,
    const int* __restrict__ cu_k, int kv_heads, const int2* __restrict__ copies,
    const int* __restrict__ n_copy, int k_sel, int pool_slots, bf16_t* __restrict__ kpool,
    bf16_t* __restrict__ vpool) {
  const int j = blockIdx.x;
  const size_t unit = blockIdx.y;
  if (j >= n_copy[unit]) return;
  const int2 c = copies[unit * k_sel + j];  // (block, slot)
  const int b = int(unit / kv_heads), g = int(unit % kv_heads);
  const int kstart = cu_k[b], len = cu_k[b + 1] - kstart;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int tok = c.x * kBlock + row;
  if (c.x < 0 || tok >= len || c.y < 0 || c.y >= pool_slots) return;
  const size_t src = (size_t(kstart + tok) * kv_heads + g) * kHeadDim + 32 * part;
  const size_t dst = ((unit * pool_slots + c.y) * kBlock + row) * kHeadDim + 32 * part;
  uint4 a[4], w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ld16(k_src + src + 8 * i);
    w[i] = ld16(v_src + src + 8 * i);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint4*>(kpool + dst + 8 * i) = a[i];
    *reinterpret_cast<uint4*>(vpool + dst + 8 * i) = w[i];
  }
}

}  // namespace

hipError_t launch_offload_reset(int* slot_of, size_t n_slot_of, int* block_of, size_t n_block_of,
                                hipStream_t s) {
  hipError_t e = hipSuccess;
  if (n_slot_of > 0)
    e = launch_kernel(kKindPool, fill_neg1_kernel,
                      dim3(unsigned(std::min<size_t>((n_slot_of + 255) / 256, 4096))), dim3(256), s,
                      slot_of, n_slot_of);
  if (e != hipSuccess || n_block_of == 0) return e;
  return launch_kernel(kKindPool, fill_neg1_kernel,
                       dim3(unsigned(std::min<size_t>((n_block_of + 255) / 256, 4096))), dim3(256), s,
                       block_of, n_block_of);
}

hipError_t launch_offload_fetch(const OffloadArgs& a, hipStream_t s) {
  hipError_t e = launch_kernel(kKindBlockScores, offload_plan_kernel, dim3(a.units),
                               dim3(kPlanThreads), s, a.indices, a.k_sel, a.slot_of, a.nb_cap,
                               a.block_of, a.pool_slots, a.slot_ids, a.copies, a.n_copy,
                               a.fetched);
  if (e != hipSuccess) return e;
  return launch_kernel(kKindFetch, offload_fetch_kernel, dim3(a.k_sel, a.units), dim3(256), s,
                       a.k_src, a.v_src, a.cu_k, a.kv_heads,
                       static_cast<const int2*>(a.copies), static_cast<const int*>(a.n_copy),
                       a.k_sel, a.pool_slots, a.kpool, a.vpool);
}

}  // namespace nsa
