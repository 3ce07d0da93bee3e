// nsa_decode_step_noalloc: the decode step with its workspace in a fixed device
// array owned by the library, for callers that must not allocate (code under
// stream capture, serving loops that forbid allocation).  The kernels are those
// of nsa_decode_step; only where the workspace comes from differs.
#include <cstdio>
#include <mutex>

#include "../../include/nsa.h"
#include "launch.h"

namespace nsa {
nsa_status set_error(nsa_status st, const char* msg);  // api.hip: the nsa_last_error text
}

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

// Per-device scratch: each GPU that loads the library holds its own copy until
// the process ends.  Host code never passes this name to a kernel (on the host
// it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the device in question.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current.
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t nsa_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

nsa_status nsa_decode_step_noalloc(const nsa_decode_params* p, hipStream_t stream) {
  // argument checks and the workspace size are those of the allocating entry point
  const size_t need = nsa_decode_workspace_size(p);
  if (need == 0) return nsa_decode_step(p, nullptr, 0, stream);  // empty batch or bad arguments
  char msg[256];
  if (need > kScratchBytes) {
    std::snprintf(msg, sizeof(msg),
                  "nsa_decode_step_noalloc: this step needs %zu bytes of workspace, above the "
                  "fixed scratch of %zu bytes (use nsa_decode_step with a caller workspace)",
                  need, kScratchBytes);
    return nsa::set_error(NSA_ERR_WORKSPACE, msg);
  }
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nsa::set_error(NSA_ERR_HIP, "nsa_decode_step_noalloc: no usable device for the stream");
  void* ws = nullptr;
  if ((e = scratch_on(dev, &ws)) != hipSuccess) {
    std::snprintf(msg, sizeof(msg), "nsa_decode_step_noalloc: scratch address lookup failed: %s",
                  hipGetErrorString(e));
    return nsa::set_error(NSA_ERR_HIP, msg);
  }
  return nsa_decode_step(p, ws, kScratchBytes, stream);
}

}  // extern "C"
