// Per-kernel-class event timing used by the C ABI (see li_timing_enable).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/latentindex.h"

namespace li {

// Brackets the launches issued during its lifetime when timing is enabled.
class TimedScope {
  public:
    TimedScope(int cls, hipStream_t s);
    ~TimedScope();
    TimedScope(const TimedScope &) = delete;
    TimedScope &operator=(const TimedScope &) = delete;

  private:
    int cls_;
    hipStream_t s_;
    hipEvent_t a_, b_;
};

void timing_enable(bool on);
hipError_t timing_read(int cls, double *total_ms, int64_t *launches);

} // namespace li
