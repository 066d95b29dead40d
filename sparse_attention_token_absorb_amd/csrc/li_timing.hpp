// Per-kernel-class event timing used by the C ABI (see li_timing_enable).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/latentindex.h"

namespace li {

// Brackets the launches issued during its lifetime when timing is enabled.
// A one-kernel scope holds exactly one launch made through launch_kernel:
// that launch binds the scope's events to the kernel's own start and end, so
// the interval leaves out the dispatch of the kernel after the stream's
// preceding work.  Any other scope records its events on the stream around
// whatever it launches.
class TimedScope {
  public:
    TimedScope(int cls, hipStream_t s, bool one_kernel = false);
    ~TimedScope();
    TimedScope(const TimedScope &) = delete;
    TimedScope &operator=(const TimedScope &) = delete;

  private:
    friend void kernel_events(hipEvent_t *start, hipEvent_t *stop);
    int cls_;
    hipStream_t s_;
    hipEvent_t a_, b_;
    bool one_, taken_;
    TimedScope *prev_;
};

// The events the next launch binds to its kernel: the enclosing one-kernel
// scope's pair, once; null (an untimed launch) otherwise.
void kernel_events(hipEvent_t *start, hipEvent_t *stop);

// A kernel launch that a one-kernel TimedScope can time.
template <typename F, typename... Args>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args)
{
    hipEvent_t a = nullptr, b = nullptr;
    kernel_events(&a, &b);
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, a, b, 0u, args...);
    return hipGetLastError();
}

void timing_enable(bool on);
hipError_t timing_read(int cls, double *total_ms, int64_t *launches);

} // namespace li
