// Key sets of the backward kernels (selected blocks, sliding window, visible
// compressed windows) and the position of a packed query row; shared by the
// vector-ALU and the matrix-core backward kernels.
#pragma once

#include "common.h"
#include "launch.h"

namespace nsa {

// Row r of sequence b sits at position t = (r - cu_q[b]) + (L_b - Lq_b).
__device__ __forceinline__ void bwd_row_position(int row, const int* __restrict__ cu_q,
                                                 const int* __restrict__ cu_k, int batch, int& b,
                                                 int& t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  b = lo;
  t = (row - cu_q[b]) + ((cu_k[b + 1] - cu_k[b]) - (cu_q[b + 1] - cu_q[b]));
}

// Whether key j (a row of the key tensor, 0-based within its sequence, klen
// keys) takes part in the attention of query position t.
template <int MODE>
__device__ __forceinline__ bool key_visible(int j, int t, int klen, int window) {
  if constexpr (MODE == kBwdSelected) return j <= t;
  else if constexpr (MODE == kBwdWindow) return j <= t && j > t - window;
  else return j < klen && kStride * j + kKernel - 1 <= t;
}

// Query positions that see key block `id` of sequence b in an implicit mode:
// t_lo .. t_lo + n - 1 (clipped to the sequence's query rows, row
// cu_q[b] + t - shift); returns n.
template <int MODE>
__device__ __forceinline__ int implicit_rows(int b, int id, int klen, int window,
                                             const int* __restrict__ cu_q,
                                             const int* __restrict__ cu_k, int& t_lo,
                                             int& row_lo) {
  const int len = cu_k[b + 1] - cu_k[b];
  const int shift = len - (cu_q[b + 1] - cu_q[b]);
  int lo, hi;
  if constexpr (MODE == kBwdWindow) {
    lo = kBlock * id;
    hi = min(kBlock * id + kBlock - 1, klen - 1) + window - 1;
  } else {
    lo = kStride * (kBlock * id) + kKernel - 1;
    hi = len - 1;
  }
  lo = max(lo, shift);
  hi = min(hi, len - 1);
  t_lo = lo;
  row_lo = cu_q[b] + lo - shift;
  return max(0, hi - lo + 1);
}

}  // namespace nsa
