// Debug mode: device-side checks of the preconditions the release path takes on
// trust (the varlen batch layout, unique block ids per index row, NaN-free
// block scores).  Off by default; nsa_set_debug_checks(1) turns it on for the
// process.  While on, an entry point first launches the checks that apply to
// its arguments on the caller's stream, then waits for them (this is the one
// place the library synchronises) and returns NSA_ERR_INVALID_ARG, without
// launching its work, when one fails.
//
// The sequence layout checked is the one the pages' varlen kernels rely on
// (NOSA-1B source analysis part 3, the variable-length mask: sequence b spans
// rows cu[b] .. cu[b+1]-1 of the packed tensor); unique ids follow the block
// lists of TileLang NSA, section 2.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <mutex>

#include "checks.h"
#include "common.h"

namespace nsa {

namespace {

// One flag word per device: bit i set = check kind i failed.  Device memory of
// the library (no allocation per call); its address is looked up once per
// device.
static __device__ __align__(16) int check_flags[4];

constexpr int kMaxCheckDevices = 64;
std::mutex g_mu;
int* g_flags[kMaxCheckDevices] = {};
std::atomic<int> g_enabled{0};

__global__ void clear_flags_kernel(int* flags) {
  if (threadIdx.x < 4) flags[threadIdx.x] = 0;
}

// cu[0] == 0, cu non-decreasing, every length <= max_len (max_len < 0: no bound).
__global__ __launch_bounds__(256) void check_cu_kernel(const int* __restrict__ cu, int batch,
                                                       int max_len, int bit,
                                                       int* __restrict__ flags) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b > batch) return;
  bool bad = false;
  if (b == 0) bad = cu[0] != 0;
  else {
    const int len = cu[b] - cu[b - 1];
    bad = len < 0 || (max_len >= 0 && len > max_len);
  }
  if (bad) atomicOr(flags, 1 << bit);
}

// Per sequence: count_c[b] <= windows covering count[b] tokens (the pooling and
// scoring paths never need more windows than cover the sequence).
__global__ __launch_bounds__(256) void check_windows_kernel(const int* __restrict__ cu,
                                                            const int* __restrict__ cu_c,
                                                            int batch, int kernel, int stride,
                                                            int* __restrict__ flags) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  const int len = cu[b + 1] - cu[b], nc = cu_c[b + 1] - cu_c[b];
  int cover = 0;
  if (len > 0) cover = len <= kernel ? 1 : (len - kernel + stride - 1) / stride + 1;
  if (nc < 0 || nc > cover) atomicOr(flags, 1 << kCheckWindows);
}

// One thread per index row: the non-negative ids of the row are distinct.
__global__ __launch_bounds__(256) void check_unique_kernel(const int* __restrict__ idx,
                                                           long rows, int k,
                                                           int* __restrict__ flags) {
  const long r = long(blockIdx.x) * 256 + threadIdx.x;
  if (r >= rows) return;
  const int* row = idx + r * k;
  for (int i = 0; i < k; ++i) {
    const int a = row[i];
    if (a < 0) continue;
    for (int j = i + 1; j < k; ++j)
      if (row[j] == a) {
        atomicOr(flags, 1 << kCheckUniqueIds);
        return;
      }
  }
}

// Per sequence: query rows <= keys (a query row sits at a key position).
__global__ __launch_bounds__(256) void check_q_within_k_kernel(const int* __restrict__ cu_q,
                                                               const int* __restrict__ cu_k,
                                                               int batch, int* __restrict__ flags) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  if (cu_q[b + 1] - cu_q[b] > cu_k[b + 1] - cu_k[b]) atomicOr(flags, 1 << kCheckQWithinK);
}

__global__ __launch_bounds__(256) void check_nan_kernel(const float* __restrict__ x, long n,
                                                        int* __restrict__ flags) {
  for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n; i += long(gridDim.x) * 256)
    if (x[i] != x[i]) {
      atomicOr(flags, 1 << kCheckNaN);
      return;
    }
}

const char* kind_text(int bits) {
  if (bits & (1 << kCheckCuK)) return "cu_seqlens_k is not a valid offset array (cu[0] != 0, decreasing, or a sequence longer than max_seqlen_k)";
  if (bits & (1 << kCheckCuQ)) return "cu_seqlens_q is not a valid offset array (cu[0] != 0 or decreasing)";
  if (bits & (1 << kCheckCuC)) return "cu_seqlens_c is not a valid offset array";
  if (bits & (1 << kCheckWindows)) return "a sequence has more windows in cu_seqlens_c than cover its tokens";
  if (bits & (1 << kCheckUniqueIds)) return "an index row lists the same block id twice";
  if (bits & (1 << kCheckNaN)) return "the block scores hold a NaN";
  if (bits & (1 << kCheckQWithinK)) return "a sequence has more query rows than keys";
  return "unknown check";
}

}  // namespace

bool debug_checks_on() { return g_enabled.load(std::memory_order_relaxed) != 0; }

int set_debug_checks(int on) { return g_enabled.exchange(on ? 1 : 0); }

DebugChecks::DebugChecks(hipStream_t s) : s_(s) {
  int dev = -1;
  hipError_t e = s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxCheckDevices) {
    err_ = e != hipSuccess ? e : hipErrorInvalidDevice;
    return;
  }
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_flags[dev] == nullptr) {
      int cur = -1;
      if ((e = hipGetDevice(&cur)) != hipSuccess) { err_ = e; return; }
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) { err_ = e; return; }
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flags));
      if (cur != dev) hipSetDevice(cur);
      if (e != hipSuccess) { err_ = e; return; }
      g_flags[dev] = static_cast<int*>(p);
    }
    flags_ = g_flags[dev];
  }
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, s_, flags_);
  err_ = hipGetLastError();
}

void DebugChecks::cu(const int* cu, int batch, int max_len, int bit) {
  if (err_ != hipSuccess || cu == nullptr || batch < 0) return;
  hipLaunchKernelGGL(check_cu_kernel, dim3(unsigned(batch / 256 + 1)), dim3(256), 0, s_, cu, batch,
                     max_len, bit, flags_);
  err_ = hipGetLastError();
}

void DebugChecks::q_within_k(const int* cu_q, const int* cu_k, int batch) {
  if (err_ != hipSuccess || cu_q == nullptr || cu_k == nullptr || batch <= 0) return;
  hipLaunchKernelGGL(check_q_within_k_kernel, dim3(unsigned((batch + 255) / 256)), dim3(256), 0,
                     s_, cu_q, cu_k, batch, flags_);
  err_ = hipGetLastError();
}

void DebugChecks::windows(const int* cu, const int* cu_c, int batch, int kernel, int stride) {
  if (err_ != hipSuccess || cu == nullptr || cu_c == nullptr || batch <= 0) return;
  hipLaunchKernelGGL(check_windows_kernel, dim3(unsigned((batch + 255) / 256)), dim3(256), 0, s_,
                     cu, cu_c, batch, kernel, stride, flags_);
  err_ = hipGetLastError();
}

void DebugChecks::unique_ids(const int* idx, long rows, int k) {
  if (err_ != hipSuccess || idx == nullptr || rows <= 0 || k <= 0) return;
  hipLaunchKernelGGL(check_unique_kernel, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, s_,
                     idx, rows, k, flags_);
  err_ = hipGetLastError();
}

void DebugChecks::no_nan(const float* x, long n) {
  if (err_ != hipSuccess || x == nullptr || n <= 0) return;
  const long blocks = std::min<long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(check_nan_kernel, dim3(unsigned(blocks)), dim3(256), 0, s_, x, n, flags_);
  err_ = hipGetLastError();
}

bool DebugChecks::failed(char* msg, size_t msg_len) {
  if (err_ == hipSuccess) err_ = hipStreamSynchronize(s_);
  int bits = 0;
  if (err_ == hipSuccess) err_ = hipMemcpy(&bits, flags_, sizeof(int), hipMemcpyDeviceToHost);
  if (err_ != hipSuccess) {
    std::snprintf(msg, msg_len, "device checks could not run: %s", hipGetErrorString(err_));
    return true;
  }
  if (bits == 0) return false;
  std::snprintf(msg, msg_len, "device check failed: %s", kind_text(bits));
  return true;
}

}  // namespace nsa
