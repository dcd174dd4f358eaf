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

// Loss options shared by every launch of one call.
enum class Reduction { Mean = 0, Sum = 1, None = 2 };
struct LossOpts {
  int ignore = -100;
  float eps = 0.0f;     // label smoothing
  float zloss = 0.0f;   // alpha of the z-loss term alpha * LSE^2
  Reduction reduction = Reduction::Mean;
};

// `grad`: the upstream gradient, a device scalar (mean / sum) or NULL (1).
hipError_t launch_label_scan(const Plan& p, const int32_t* labels, const LossOpts& o,
                             const float* grad, char* ws, hipStream_t st, KernelTimer* timer);

// `loss`: one float (mean / sum) or N floats (none).
hipError_t launch_forward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                          const LossOpts& o, float* loss, float* lse, char* ws, hipStream_t st,
                          KernelTimer* timer);

// `grad_tok`: per-token upstream gradient [N] for reduction none, or NULL (1).
hipError_t launch_backward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                           const LossOpts& o, const float* lse, const float* grad_tok, float* dX,
                           float* dW, char* ws, hipStream_t st, KernelTimer* timer);

}  // namespace fce
