// Optional per-kernel timing with HIP events (diagnostics for roofline reports).
#pragma once

#include <hip/hip_runtime.h>

namespace tpconv {

// Kernel classes; the numbering matches tpconv_kernel in include/tpconv.h.
enum KernelClass : int {
  kcStreamFwd = 0, kcStreamJvp, kcStreamSnd, kcStreamSndT, kcStreamBwdPos,
  kcGemmOut, kcGemmGs, kcGemmGx, kcGemmGw, kcGwReduce, kcFill, kcGraph,
  kcCwContract, kcCwGw, kcCwReduce, kcStreamHess, kcStateDot, kcCount
};

// While timing is enabled, brackets the launches issued in its lifetime with
// two events on stream s; otherwise does nothing.
class TimingScope {
 public:
  TimingScope(int cls, hipStream_t s);
  ~TimingScope();
  TimingScope(const TimingScope&) = delete;
  TimingScope& operator=(const TimingScope&) = delete;

 private:
  int cls_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr;
};

bool timing_set(bool enable);  // clears the table; returns false on a HIP error
bool timing_enabled();
bool timing_read(int cls, long long* launches, double* total_ms);

}  // namespace tpconv
