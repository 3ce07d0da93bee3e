// Device helpers shared by the gfx950 kernels: bf16 packing, wave reductions,
// vector loads.  Wavefronts are 64 lanes wide on CDNA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct bf16_t {
  uint16_t bits;
};

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// v_dot2_f32_bf16: acc + a.lo*b.lo + a.hi*b.hi, products exact, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ------------------------------------------------------------------ loads

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 8 consecutive elements as floats.
__device__ __forceinline__ void load8f(const float* p, float* o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8f(const bf16_t* p, float* o) {
  uint4 a = ld16(p);
  o[0] = bf16lo(a.x); o[1] = bf16hi(a.x); o[2] = bf16lo(a.y); o[3] = bf16hi(a.y);
  o[4] = bf16lo(a.z); o[5] = bf16hi(a.z); o[6] = bf16lo(a.w); o[7] = bf16hi(a.w);
}

// 4 consecutive elements as floats.
__device__ __forceinline__ void load4f(const float* p, float* o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void load4f(const bf16_t* p, float* o) {
  uint2 a = *reinterpret_cast<const uint2*>(p);
  o[0] = bf16lo(a.x); o[1] = bf16hi(a.x); o[2] = bf16lo(a.y); o[3] = bf16hi(a.y);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ void store_f32(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_f32(bf16_t* p, float x) { p->bits = f32_to_bf16(x); }

// --------------------------------------------------------------- reductions
//
// Cross-lane steps use DPP row operations and the gfx950 row-pair swaps, all of
// them VALU instructions (no LDS round trip): within a row of 16 lanes
// quad_perm / row_half_mirror / row_mirror / row_ror, across rows
// v_permlane16_swap (rows 0<->1, 2<->3) and v_permlane32_swap (lanes L<->L^32).

enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
  kDppRowRor2 = 0x122,
  kDppRowRor4 = 0x124,
  kDppRowRor8 = 0x128,
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}

// For a commutative op the two swap results together are {own, partner}, so
// op(r0, r1) = op(own, partner) with no select needed.
template <typename Op>
__device__ __forceinline__ float cross16(float x, Op op) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float cross32(float x, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ int cross16i(int x, Op op) {
  auto r = __builtin_amdgcn_permlane16_swap(unsigned(x), unsigned(x), false, false);
  return op(int(r[0]), int(r[1]));
}
template <typename Op>
__device__ __forceinline__ int cross32i(int x, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(unsigned(x), unsigned(x), false, false);
  return op(int(r[0]), int(r[1]));
}

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMinI {
  __device__ __forceinline__ int operator()(int a, int b) const { return min(a, b); }
};

// Reduction over the 4 lanes of a quad (result in all 4).
template <typename Op>
__device__ __forceinline__ float quad_reduce(float x, Op op) {
  x = op(x, dpp<kDppQuadXor1>(x));
  return op(x, dpp<kDppQuadXor2>(x));
}
// Reduction over a row of 16 lanes (result in all 16).
template <typename Op>
__device__ __forceinline__ float row_reduce(float x, Op op) {
  x = quad_reduce(x, op);
  x = op(x, dpp<kDppRowHalfMirror>(x));
  return op(x, dpp<kDppRowMirror>(x));
}
// Reduction over the whole wave (result in all 64 lanes).
template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = row_reduce(x, op);
  x = cross16(x, op);
  return cross32(x, op);
}
__device__ __forceinline__ float wave_max(float x) { return wave_reduce(x, OpMax()); }
// Unsigned minimum / maximum over the whole wave (result in all 64 lanes).
struct OpUMin {
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct OpUMax {
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
  x = op(x, uint32_t(dpp<kDppQuadXor1>(int(x))));
  x = op(x, uint32_t(dpp<kDppQuadXor2>(int(x))));
  x = op(x, uint32_t(dpp<kDppRowHalfMirror>(int(x))));
  x = op(x, uint32_t(dpp<kDppRowMirror>(int(x))));
  auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r16[0], r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return wave_reduce_u32(x, OpUMin()); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) { return wave_reduce_u32(x, OpUMax()); }

// Integer minimum over the whole wave (result in all 64 lanes).
__device__ __forceinline__ int wave_min_i(int x) {
  const OpMinI op;
  x = op(x, dpp<kDppQuadXor1>(x));
  x = op(x, dpp<kDppQuadXor2>(x));
  x = op(x, dpp<kDppRowHalfMirror>(x));
  x = op(x, dpp<kDppRowMirror>(x));
  x = cross16i(x, op);
  return cross32i(x, op);
}
__device__ __forceinline__ float wave_sum(float x) { return wave_reduce(x, OpSum()); }

// Inclusive prefix sum over the wave (lane order), 6 DPP / swap steps.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
  // within rows: shift-right by 1, 2, 4, 8 with zero fill
  int y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += y;
  // across rows: add the totals of all earlier rows
  const int r15 = __builtin_amdgcn_readlane(x, 15), r31 = __builtin_amdgcn_readlane(x, 31),
            r47 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  x += (row >= 1 ? r15 : 0) + (row >= 2 ? r31 : 0) + (row >= 3 ? r47 : 0);
  return x;
}

// The workgroups of a launch are handed to the 8 XCDs in turn (launch-order id
// modulo 8), and each XCD has its own L2.  This maps a launch-order id of a
// one-dimensional grid of `total` workgroups to a logical index such that every
// XCD takes one contiguous range of logical indices: workgroups with
// neighbouring logical indices (the splits or chunks of one sequence and KV
// head) then share one XCD and its L2.  A bijection on [0, total).
__device__ __forceinline__ int xcd_grouped_index(int id, int total) {
  const int x = id & 7, j = id >> 3, q = total >> 3, r = total & 7;
  return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// exp2 on the hardware unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map float -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace nsa
