// Sliding-window mean pooling over packed variable-length sequences.
//
// One kernel serves the key compressor (NOSA-1B core components, component 1:
// 32-token windows, stride 16, one mean per window) and the CIS pooling kernel
// (NOSA-1B source analysis part 3: a program per (head, batch, window), a masked
// load of the window, the sum divided by the count of valid tokens).  A thread
// owns VEC consecutive channels of one row, so the lanes of a wave read whole
// token rows with 16-byte loads; the launch is a 2-D grid (run of windows x
// channel slot, sequence).
// When the window is two strides long (32/16), every token is read once: a
// thread sums one stride-long half of the windows in token order into LDS, and
// window c is half c plus half c+1 divided by its count of valid tokens.  Other
// geometries sum each window's tokens in order.
#include "common.h"
#include "launch.h"

namespace nsa {

template <typename T, int VEC>
struct VecIO;

template <>
struct VecIO<bf16_t, 8> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* x) { load8f(p, x); }
};

template <>
struct VecIO<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    float4 a = *reinterpret_cast<const float4*>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
};

template <typename T>
struct VecIO<T, 1> {
  static __device__ __forceinline__ void load(const T* p, float* x) { x[0] = to_f32(*p); }
};

// Output store of VEC floats into Tout.
template <typename Tout, int VEC>
__device__ __forceinline__ void store_vec(Tout* p, const float* v) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) store_f32(p + e, v[e]);
}
template <>
__device__ __forceinline__ void store_vec<bf16_t, 8>(bf16_t* p, const float* v) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = w;
}
template <>
__device__ __forceinline__ void store_vec<float, 4>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename Tin, typename Tout, int VEC>
__global__ __launch_bounds__(256) void mean_pool_kernel(const Tin* __restrict__ x,
                                                        Tout* __restrict__ y,
                                                        const int* __restrict__ cu,
                                                        const int* __restrict__ cuc, int width,
                                                        int kernel, int stride, int last_n) {
  const int b = blockIdx.y;
  const int start = cu[b];
  const int len = cu[b + 1] - start;
  const int cbase = cuc[b];
  const int nc = cuc[b + 1] - cbase;
  const int tpw = width / VEC;  // threads per window row
  const long gid = long(blockIdx.x) * blockDim.x + threadIdx.x;
  int c = int(gid / tpw);
  const int slot = int(gid - long(c) * tpw);
  if (last_n > 0) c += max(0, nc - last_n);
  if (c >= nc) return;
  const int lo = stride * c;
  const int hi = min(lo + kernel, len);
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const Tin* src = x + (size_t(start) + lo) * width + size_t(slot) * VEC;
  // tokens are summed in order; the loads of 8 tokens are issued together
  int j = lo;
  for (; j + 8 <= hi; j += 8, src += 8 * size_t(width)) {
    float xs[8][VEC];
#pragma unroll
    for (int u = 0; u < 8; ++u) VecIO<Tin, VEC>::load(src + size_t(u) * width, xs[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += xs[u][e];
  }
  for (; j < hi; ++j, src += width) {
    float xs[VEC];
    VecIO<Tin, VEC>::load(src, xs);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += xs[e];
  }
  const int n = hi - lo;
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = n > 0 ? acc[e] / float(n) : 0.f;
  store_vec<Tout, VEC>(y + (size_t(cbase) + c) * width + size_t(slot) * VEC, acc);
}

// Windows two strides long: workgroup of 512 threads, kHalves = 512 / tpw halves
// of `stride` tokens (tpw threads per row), windows c0 .. c0 + kHalves - 2.
template <typename Tin, typename Tout, int VEC>
__global__ __launch_bounds__(512) void mean_pool_halves_kernel(const Tin* __restrict__ x,
                                                               Tout* __restrict__ y,
                                                               const int* __restrict__ cu,
                                                               const int* __restrict__ cuc,
                                                               int width, int stride, int last_n) {
  __shared__ float hs[512 * VEC];  // [half][slot][e]
  const int b = blockIdx.y;
  const int start = cu[b];
  const int len = cu[b + 1] - start;
  const int cbase = cuc[b];
  const int nc = cuc[b + 1] - cbase;
  const int tpw = width / VEC;
  const int halves = 512 / tpw;  // >= 2 (host-checked)
  const int c0 = int(blockIdx.x) * (halves - 1) + (last_n > 0 ? max(0, nc - last_n) : 0);
  if (c0 >= nc) return;  // whole workgroup
  const int hh = int(threadIdx.x) / tpw, slot = int(threadIdx.x) % tpw;
  if (hh < halves) {
    // half c0 + hh: tokens stride*(c0+hh) .. +stride-1 that exist, summed in order
    const int lo = stride * (c0 + hh);
    const int hi = min(lo + stride, len);
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    const Tin* src = x + (size_t(start) + lo) * width + size_t(slot) * VEC;
    int j = lo;
    for (; j + 8 <= hi; j += 8, src += 8 * size_t(width)) {
      float xs[8][VEC];
#pragma unroll
      for (int u = 0; u < 8; ++u) VecIO<Tin, VEC>::load(src + size_t(u) * width, xs[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += xs[u][e];
    }
    for (; j < hi; ++j, src += width) {
      float xs[VEC];
      VecIO<Tin, VEC>::load(src, xs);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += xs[e];
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) hs[(hh * tpw + slot) * VEC + e] = acc[e];
  }
  __syncthreads();
  const int c = c0 + hh;
  if (hh < halves - 1 && c < nc) {
    const int n = max(0, min(2 * stride, len - stride * c));
    float out[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float sum = hs[(hh * tpw + slot) * VEC + e] + hs[((hh + 1) * tpw + slot) * VEC + e];
      out[e] = n > 0 ? sum / float(n) : 0.f;
    }
    store_vec<Tout, VEC>(y + (size_t(cbase) + c) * width + size_t(slot) * VEC, out);
  }
}

template <typename Tin, typename Tout, int VEC>
static hipError_t launch_pool_t(const void* x, void* y, const int* cu, const int* cuc, int batch,
                                int windows, int width, int kernel, int stride, int last_n,
                                hipStream_t s) {
  if (windows == 0 || batch == 0) return hipSuccess;
  const int tpw = width / VEC;
  if (kernel == 2 * stride && tpw <= 256) {
    const int per_block = 512 / tpw - 1;  // windows per workgroup
    dim3 grid((windows + per_block - 1) / per_block, batch);
    return launch_kernel(kKindPool, mean_pool_halves_kernel<Tin, Tout, VEC>, grid, dim3(512), s,
                         static_cast<const Tin*>(x), static_cast<Tout*>(y), cu, cuc, width,
                         stride, last_n);
  }
  const long threads = long(windows) * tpw;
  const int blocks = int((threads + 255) / 256);
  dim3 grid(blocks, batch);
  return launch_kernel(kKindPool, mean_pool_kernel<Tin, Tout, VEC>, grid, dim3(256), s,
                       static_cast<const Tin*>(x), static_cast<Tout*>(y), cu, cuc, width, kernel,
                       stride, last_n);
}

hipError_t launch_mean_pool(const void* x, int x_bf16, void* y, int y_bf16, const int* cu,
                            const int* cuc, int batch, int max_windows, int width, int kernel,
                            int stride, int last_n, hipStream_t s) {
  const int windows = last_n > 0 ? last_n : max_windows;
  if (x_bf16) {
    if (y_bf16) {
      if (width % 8 == 0)
        return launch_pool_t<bf16_t, bf16_t, 8>(x, y, cu, cuc, batch, windows, width, kernel,
                                                stride, last_n, s);
      return launch_pool_t<bf16_t, bf16_t, 1>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                              last_n, s);
    }
    if (width % 8 == 0)
      return launch_pool_t<bf16_t, float, 8>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                             last_n, s);
    return launch_pool_t<bf16_t, float, 1>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                           last_n, s);
  }
  if (y_bf16) {
    if (width % 4 == 0)
      return launch_pool_t<float, bf16_t, 4>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                             last_n, s);
    return launch_pool_t<float, bf16_t, 1>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                           last_n, s);
  }
  if (width % 4 == 0)
    return launch_pool_t<float, float, 4>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                          last_n, s);
  return launch_pool_t<float, float, 1>(x, y, cu, cuc, batch, windows, width, kernel, stride,
                                        last_n, s);
}

}  // namespace nsa
