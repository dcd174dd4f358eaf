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
// use_stats: fp32 takes its exponents from the split row statistics the
// forward left in this workspace (the fused call); otherwise from lse alone.
hipError_t launch_backward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                           const LossOpts& o, const float* lse, bool use_stats,
                           const float* grad_tok, float* dX, float* dW, char* ws, hipStream_t st,
                           KernelTimer* timer);

// Store-logits variant of forward + backward (upstream gradient 1): the plan
// must be made with Variant::StoreLogits; the label scan runs first.
hipError_t launch_fused_store(const Plan& p, const void* X, const void* W, const int32_t* labels,
                              const LossOpts& o, float* loss, float* lse, float* dX, float* dW,
                              char* ws, hipStream_t st, KernelTimer* timer);

// Loss (and optionally dZ) on logits the caller holds.  Workspace layout:
// Ctrl, one flag word, then N per-row loss terms (each 256-byte aligned).
constexpr size_t ce_off_ctrl() { return 0; }
constexpr size_t ce_off_flags() { return 256; }
constexpr size_t ce_off_rowloss() { return 512; }
inline size_t ce_workspace_bytes(int64_t N) {
  return ce_off_rowloss() + ((static_cast<size_t>(std::max<int64_t>(N, 1)) * 4 + 255) / 256) * 256;
}
struct CeLogitsCall {
  const void* Z;
  int64_t ldz;
  void* dZ;  // may equal Z, or NULL
  int64_t lddz;
  const int32_t* labels;
  int64_t N, V;
  bool bf16;
  LossOpts o;
  const float* grad;  // scalar (mean / sum) or per-token (none), or NULL
  float* loss;        // [1] or [N] (none)
  float* lse;         // [N]
  char* ws;
};
hipError_t launch_ce_logits(const CeLogitsCall& c, hipStream_t st, KernelTimer* timer);

// The current device's copy of the library's static scratch
// (FCE_STATIC_SCRATCH_BYTES), looked up on the first call per device.
hipError_t static_scratch(void** ptr, size_t* bytes);

// dX[0 .. n_dx) and dW[0 .. n_dw) multiplied in place by the device scalar g.
hipError_t launch_scale_grads(float* dX, int64_t n_dx, float* dW, int64_t n_dw, const float* g,
                              hipStream_t st, KernelTimer* timer);

}  // namespace fce
