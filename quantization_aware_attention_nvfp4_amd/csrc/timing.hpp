// timing.hpp - event bracketing of kernel launches while aq_kernel_timing(1) is in effect.
#pragma once

#include <hip/hip_runtime.h>

namespace aq {

bool timing_on();
void timing_begin(hipEvent_t *start, hipStream_t stream);
void timing_end(const char *name, hipEvent_t start, hipStream_t stream);

}  // namespace aq

// Launch a kernel; when timing is on, bracket it with events recorded on its stream.
#define AQ_LAUNCH(name, kernel, grid, block, smem, stream, ...)                         \
  do {                                                                                  \
    hipEvent_t aq_t0_ = nullptr;                                                        \
    const bool aq_timed_ = ::aq::timing_on();                                           \
    if (aq_timed_) ::aq::timing_begin(&aq_t0_, (stream));                               \
    hipLaunchKernelGGL(kernel, grid, block, smem, stream, __VA_ARGS__);                 \
    if (aq_timed_) ::aq::timing_end(name, aq_t0_, (stream));                            \
  } while (0)
