// Internal C++ interface between the C ABI (fce_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <algorithm>

#include "fce_plan.h"

namespace fce {

// Optional per-kernel event timing (see fce_timing_enable in fce.h).
class KernelTimer {
 public:
  virtual ~KernelTimer() = default;
  virtual void begin(const char* name, double flops, hipStream_t st) = 0;
  virtual void end(hipStream_t st) = 0;
};

hipError_t launch_label_scan(const Plan& p, const int32_t* labels, int ignore, int reduction_sum,
                             const float* grad, char* ws, hipStream_t st, KernelTimer* timer);

hipError_t launch_forward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                          int ignore, float eps, float* loss, float* lse, char* ws, hipStream_t st,
                          KernelTimer* timer);

hipError_t launch_backward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                           int ignore, float eps, const float* lse, float* dX, float* dW, char* ws,
                           hipStream_t st, KernelTimer* timer);

}  // namespace fce
