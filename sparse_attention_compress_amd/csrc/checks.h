// Debug-mode device checks of the preconditions (see checks.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace nsa {

enum CheckKind {
  kCheckCuK = 0,        // key offsets
  kCheckCuQ = 1,        // query-row offsets
  kCheckCuC = 2,        // window offsets
  kCheckWindows = 3,    // window count of a sequence
  kCheckUniqueIds = 4,  // block ids of one index row
  kCheckNaN = 5,        // block scores
  kCheckQWithinK = 6,   // query rows of a sequence <= its keys
};

bool debug_checks_on();
int set_debug_checks(int on);

// The checks of one entry point: construct on the call's stream, add checks,
// then failed() waits for them and says whether any precondition is broken.
class DebugChecks {
 public:
  explicit DebugChecks(hipStream_t s);
  void cu(const int* cu, int batch, int max_len, int bit);
  void q_within_k(const int* cu_q, const int* cu_k, int batch);
  void windows(const int* cu, const int* cu_c, int batch, int kernel, int stride);
  void unique_ids(const int* idx, long rows, int k);
  void no_nan(const float* x, long n);
  bool failed(char* msg, size_t msg_len);

 private:
  hipStream_t s_;
  int* flags_ = nullptr;
  hipError_t err_ = hipSuccess;
};

}  // namespace nsa
