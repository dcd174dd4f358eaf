// C ABI of the fused linear cross-entropy library: argument validation,
// planning, and the launch sequences of fce_forward / fce_backward /
// fce_fused_fwd_bwd.  Nothing here allocates device memory.
#include "fce.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fce_kernels.h"
#include "fce_plan.h"

namespace {

// Last HIP error a library call of this thread ran into (for
// fce_last_hip_error); hipSuccess until one does.
thread_local hipError_t t_last_hip = hipSuccess;

fce_status from_hip(hipError_t e) {
  if (e == hipSuccess) return FCE_OK;
  t_last_hip = e;
  return FCE_ERR_HIP;
}

using fce::Dtype;
using fce::Plan;
using fce::Schedule;

// --------------------------------------------------------------- timing
// Kernel durations from HIP events on the caller's stream.  Within one call
// the timed launches follow each other with nothing between them, so a
// launch's start is the previous launch's stop: one event per boundary
// (each record on the stream costs a few microseconds of its time).  Every
// entry point calls new_call() first, so work the caller enqueues between
// calls never falls inside a timed interval.
struct Record {
  std::string name;
  double flops;
  int start, stop;  // event indices
};

// Events created when timing is switched on: about 25 kernel boundaries per
// fused call at the largest plans, for 40 calls between reads.
constexpr size_t kTimerPreallocEvents = 1024;

class EventTimer final : public fce::KernelTimer {
 public:
  bool enabled = false;
  std::vector<hipEvent_t> pool;
  int used = 0;            // events recorded since the last read
  std::vector<Record> records;
  int open = -1;           // record waiting for its stop event
  int last_stop = -1;      // stop event of the previous launch of this call
  hipStream_t last_stream = nullptr;
  bool failed = false;

  void new_call() { last_stop = -1; }
  int next_event() {
    if (used >= static_cast<int>(pool.size())) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) {
        failed = true;
        return -1;
      }
      pool.push_back(e);
    }
    return used++;
  }
  void begin(const char* name, double flops, hipStream_t st) override {
    if (!enabled) return;
    int start = (last_stop >= 0 && st == last_stream) ? last_stop : -1;
    if (start < 0) {
      start = next_event();
      if (start < 0) return;
      if (hipEventRecord(pool[start], st) != hipSuccess) failed = true;
    }
    records.push_back(Record{name, flops, start, -1});
    open = static_cast<int>(records.size()) - 1;
  }
  void end(hipStream_t st) override {
    if (!enabled || open < 0) return;
    const int stop = next_event();
    if (stop < 0) {
      records.pop_back();
      open = -1;
      return;
    }
    if (hipEventRecord(pool[stop], st) != hipSuccess) failed = true;
    records[open].stop = stop;
    open = -1;
    last_stop = stop;
    last_stream = st;
  }
};

class NullTimer final : public fce::KernelTimer {
 public:
  void begin(const char*, double, hipStream_t) override {}
  void end(hipStream_t) override {}
};

// Mutable global state besides the device-arch cache and the planner's plan
// cache (fce_plan.cpp): the optional kernel timer, guarded by g_timer_mu.  While timing is
// on, each entry point holds the mutex from its first launch to its last
// (TimerScope), so calls from several threads serialise their enqueueing and
// their records never interleave; with timing off no lock is taken.
EventTimer g_timer;
std::mutex g_timer_mu;
std::atomic<bool> g_timing_on{false};
NullTimer g_null_timer;
std::mutex g_arch_mu;
int g_arch_ok[64] = {0};  // 0 unknown, 1 gfx950, -1 other

// The timer of one entry-point call.  next() starts a chain of boundary
// events for one launch sequence.
class TimerScope {
 public:
  TimerScope() {
    if (g_timing_on.load(std::memory_order_acquire)) {
      lock_ = std::unique_lock<std::mutex>(g_timer_mu);
      on_ = g_timer.enabled;
    }
  }
  fce::KernelTimer* next() {
    if (!on_) return &g_null_timer;
    g_timer.new_call();
    return &g_timer;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  bool on_ = false;
};

fce_status check_device() {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= 64) return FCE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipError_t e = hipGetDeviceProperties(&prop, dev); e != hipSuccess) return from_hip(e);
    g_arch_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return g_arch_ok[dev] == 1 ? FCE_OK : FCE_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Which fce_variant values an entry point accepts (bit v for variant v).
constexpr unsigned kRecomputeOnly = 1u << FCE_VARIANT_RECOMPUTE;
constexpr unsigned kSplitCalls = kRecomputeOnly | (1u << FCE_VARIANT_FILTERED);
constexpr unsigned kAllVariants = kSplitCalls | (1u << FCE_VARIANT_STORE_LOGITS);

// Options of one call, checked.  allow_none: the *_ex entry points;
// variants: the fce_variant values this entry point accepts.
fce_status check_options(const fce_options* opt, bool allow_none, unsigned variants,
                         fce::LossOpts* lo) {
  if (opt == nullptr) return FCE_ERR_NULL;
  const int r = opt->reduction;
  if (r != FCE_MEAN && r != FCE_SUM && !(allow_none && r == FCE_NONE)) return FCE_ERR_ARG;
  if (opt->schedule != FCE_SCHED_AUTO && opt->schedule != FCE_SCHED_TOKEN &&
      opt->schedule != FCE_SCHED_VOCAB)
    return FCE_ERR_ARG;
  if (opt->chunk < 1) return FCE_ERR_ARG;
  if (opt->variant < 0 || opt->variant > 31 || !((variants >> opt->variant) & 1u))
    return FCE_ERR_ARG;
  const float eps = opt->label_smoothing;
  if (!(eps >= 0.0f && eps < 1.0f)) return FCE_ERR_ARG;  // also rejects NaN
  const float z = opt->z_loss;
  if (!(z >= 0.0f && z <= 3.4e38f)) return FCE_ERR_ARG;  // rejects NaN and +inf
  lo->ignore = opt->ignore_index;
  lo->eps = eps;
  lo->zloss = z;
  lo->reduction = static_cast<fce::Reduction>(r);
  return FCE_OK;
}

fce_status validate(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                    int64_t V, fce_dtype dtype, const fce_options* opt, bool allow_none,
                    unsigned variants, size_t ws_bytes, const void* ws, Plan* plan,
                    fce::LossOpts* lo) {
  if (N < 0 || H < 1 || V < 1) return FCE_ERR_SHAPE;
  if (W == nullptr || ws == nullptr) return FCE_ERR_NULL;
  if (N > 0 && (X == nullptr || labels == nullptr)) return FCE_ERR_NULL;
  if (dtype != FCE_F32 && dtype != FCE_BF16) return FCE_ERR_ARG;
  if (fce_status s = check_options(opt, allow_none, variants, lo); s != FCE_OK) return s;
  if (opt->variant == FCE_VARIANT_FILTERED && dtype != FCE_BF16) return FCE_ERR_ARG;
  const int64_t vec = (dtype == FCE_BF16) ? 8 : 4;
  if (H % vec != 0) return FCE_ERR_ALIGN;
  if (!aligned16(W) || !aligned16(ws) || (N > 0 && !aligned16(X))) return FCE_ERR_ALIGN;
  if (!fce::make_plan(N, H, V, static_cast<Dtype>(dtype), opt->chunk,
                      static_cast<Schedule>(opt->schedule), plan,
                      static_cast<fce::Variant>(opt->variant)))
    return FCE_ERR_SHAPE;
  if (ws_bytes < plan->total) return FCE_ERR_WORKSPACE;
  return FCE_OK;
}

fce_options make_options(int32_t ignore_index, float eps, fce_reduction reduction, int64_t chunk,
                         fce_schedule schedule) {
  fce_options o;
  std::memset(&o, 0, sizeof(o));
  o.ignore_index = ignore_index;
  o.label_smoothing = eps;
  o.z_loss = 0.0f;
  o.reduction = reduction;
  o.chunk = chunk;
  o.schedule = schedule;
  o.variant = 0;
  return o;
}

fce_status forward_impl(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                        int64_t V, fce_dtype dtype, const fce_options* opt, bool allow_none,
                        float* loss, float* lse, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  Plan p;
  fce::LossOpts lo;
  fce_status s = validate(X, W, labels, N, H, V, dtype, opt, allow_none,
                          allow_none ? kSplitCalls : kRecomputeOnly, workspace_bytes,
                          workspace, &p, &lo);
  if (s != FCE_OK) return s;
  const bool none = lo.reduction == fce::Reduction::None;
  if ((loss == nullptr && !(none && N == 0)) || (N > 0 && lse == nullptr)) return FCE_ERR_NULL;
  if ((s = check_device()) != FCE_OK) return s;
  char* ws = static_cast<char*>(workspace);
  TimerScope ts;
  hipError_t e = fce::launch_label_scan(p, labels, lo, nullptr, ws, stream, ts.next());
  if (e == hipSuccess)
    e = fce::launch_forward(p, X, W, labels, lo, loss, lse, ws, stream, ts.next());
  return from_hip(e);
}

fce_status backward_impl(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                         int64_t V, fce_dtype dtype, const fce_options* opt, bool allow_none,
                         const float* lse, const float* grad_loss, float* dX, float* dW,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  fce::LossOpts lo;
  fce_status s = validate(X, W, labels, N, H, V, dtype, opt, allow_none,
                          allow_none ? kSplitCalls : kRecomputeOnly, workspace_bytes,
                          workspace, &p, &lo);
  if (s != FCE_OK) return s;
  if (dW == nullptr || (N > 0 && (lse == nullptr || dX == nullptr))) return FCE_ERR_NULL;
  if (!aligned16(dW) || (N > 0 && !aligned16(dX))) return FCE_ERR_ALIGN;
  if ((s = check_device()) != FCE_OK) return s;
  const bool none = lo.reduction == fce::Reduction::None;
  char* ws = static_cast<char*>(workspace);
  TimerScope ts;
  hipError_t e = fce::launch_label_scan(p, labels, lo, none ? nullptr : grad_loss, ws, stream,
                                        ts.next());
  if (e == hipSuccess)
    e = fce::launch_backward(p, X, W, labels, lo, lse, false, none ? grad_loss : nullptr, dX,
                             dW, ws, stream, ts.next());
  return from_hip(e);
}

fce_status fused_impl(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                      int64_t V, fce_dtype dtype, const fce_options* opt, bool allow_none,
                      float* loss, float* dX, float* dW, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  Plan p;
  fce::LossOpts lo;
  fce_status s = validate(X, W, labels, N, H, V, dtype, opt, allow_none,
                          allow_none ? kAllVariants : kRecomputeOnly, workspace_bytes, workspace,
                          &p, &lo);
  if (s != FCE_OK) return s;
  const bool none = lo.reduction == fce::Reduction::None;
  if ((loss == nullptr && !(none && N == 0)) || dW == nullptr || (N > 0 && dX == nullptr))
    return FCE_ERR_NULL;
  if (!aligned16(dW) || (N > 0 && !aligned16(dX))) return FCE_ERR_ALIGN;
  if ((s = check_device()) != FCE_OK) return s;
  char* ws = static_cast<char*>(workspace);
  float* lse = reinterpret_cast<float*>(ws + p.off_lse);
  // One label scan serves both passes: with g = 1 its backward scale equals
  // the one fce_backward would compute.
  TimerScope ts;
  hipError_t e = fce::launch_label_scan(p, labels, lo, nullptr, ws, stream, ts.next());
  if (p.variant == fce::Variant::StoreLogits) {
    if (e == hipSuccess)
      e = fce::launch_fused_store(p, X, W, labels, lo, loss, lse, dX, dW, ws, stream, ts.next());
    return from_hip(e);
  }
  if (e == hipSuccess)
    e = fce::launch_forward(p, X, W, labels, lo, loss, lse, ws, stream, ts.next());
  if (e == hipSuccess)
    e = fce::launch_backward(p, X, W, labels, lo, lse, true, nullptr, dX, dW, ws, stream,
                             ts.next());
  return from_hip(e);
}

}  // namespace

extern "C" {

size_t fce_workspace_size(int64_t N, int64_t H, int64_t V, fce_dtype dtype, int64_t chunk,
                          fce_schedule schedule) {
  const fce_options o = make_options(-100, 0.0f, FCE_MEAN, chunk, schedule);
  return fce_workspace_size_ex(N, H, V, dtype, &o);
}

size_t fce_workspace_size_ex(int64_t N, int64_t H, int64_t V, fce_dtype dtype,
                             const fce_options* opt) {
  if (dtype != FCE_F32 && dtype != FCE_BF16) return 0;
  fce::LossOpts lo;
  if (check_options(opt, true, kAllVariants, &lo) != FCE_OK) return 0;
  if (opt->variant == FCE_VARIANT_FILTERED && dtype != FCE_BF16) return 0;
  Plan p;
  if (!fce::make_plan(N, H, V, static_cast<Dtype>(dtype), opt->chunk,
                      static_cast<Schedule>(opt->schedule), &p,
                      static_cast<fce::Variant>(opt->variant)))
    return 0;
  return p.total;
}

fce_status fce_plan(int64_t N, int64_t H, int64_t V, fce_dtype dtype, int64_t chunk,
                    fce_schedule schedule, fce_plan_info* out) {
  if (out == nullptr) return FCE_ERR_NULL;
  if (N < 0 || H < 1 || V < 1) return FCE_ERR_SHAPE;
  if (dtype != FCE_F32 && dtype != FCE_BF16) return FCE_ERR_ARG;
  if (schedule != FCE_SCHED_AUTO && schedule != FCE_SCHED_TOKEN && schedule != FCE_SCHED_VOCAB)
    return FCE_ERR_ARG;
  if (chunk < 1) return FCE_ERR_ARG;
  Plan p;
  if (!fce::make_plan(N, H, V, static_cast<Dtype>(dtype), chunk, static_cast<Schedule>(schedule),
                      &p))
    return FCE_ERR_SHAPE;
  out->block_tokens = p.CN;
  out->block_vocab = p.CV;
  out->n_token_blocks = p.a;
  out->n_vocab_blocks = p.b;
  out->scratch_bytes = static_cast<int64_t>(p.scratch_bytes);
  out->partial_bytes = static_cast<int64_t>(p.partial_bytes);
  out->dx_splits = p.dx_splits;
  out->workspace_bytes = static_cast<int64_t>(p.total);
  out->fwd_splits = p.fwd_splits;
  out->grad_rmw_bytes = p.grad_rmw_bytes;
  return FCE_OK;
}

fce_status fce_forward(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                       int64_t V, fce_dtype dtype, int32_t ignore_index, float label_smoothing,
                       fce_reduction reduction, int64_t chunk, fce_schedule schedule, float* loss,
                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fce_options o = make_options(ignore_index, label_smoothing, reduction, chunk, schedule);
  return forward_impl(X, W, labels, N, H, V, dtype, &o, false, loss, lse, workspace,
                      workspace_bytes, stream);
}

fce_status fce_backward(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                        int64_t V, fce_dtype dtype, int32_t ignore_index, float label_smoothing,
                        fce_reduction reduction, int64_t chunk, fce_schedule schedule,
                        const float* lse, const float* grad_loss, float* dX, float* dW,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fce_options o = make_options(ignore_index, label_smoothing, reduction, chunk, schedule);
  return backward_impl(X, W, labels, N, H, V, dtype, &o, false, lse, grad_loss, dX, dW, workspace,
                       workspace_bytes, stream);
}

fce_status fce_fused_fwd_bwd(const void* X, const void* W, const int32_t* labels, int64_t N,
                             int64_t H, int64_t V, fce_dtype dtype, int32_t ignore_index,
                             float label_smoothing, fce_reduction reduction, int64_t chunk,
                             fce_schedule schedule, float* loss, float* dX, float* dW,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fce_options o = make_options(ignore_index, label_smoothing, reduction, chunk, schedule);
  return fused_impl(X, W, labels, N, H, V, dtype, &o, false, loss, dX, dW, workspace,
                    workspace_bytes, stream);
}

fce_status fce_forward_ex(const void* X, const void* W, const int32_t* labels, int64_t N,
                          int64_t H, int64_t V, fce_dtype dtype, const fce_options* opt,
                          float* loss, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return forward_impl(X, W, labels, N, H, V, dtype, opt, true, loss, lse, workspace,
                      workspace_bytes, stream);
}

fce_status fce_backward_ex(const void* X, const void* W, const int32_t* labels, int64_t N,
                           int64_t H, int64_t V, fce_dtype dtype, const fce_options* opt,
                           const float* lse, const float* grad_loss, float* dX, float* dW,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(X, W, labels, N, H, V, dtype, opt, true, lse, grad_loss, dX, dW, workspace,
                       workspace_bytes, stream);
}

fce_status fce_fused_fwd_bwd_ex(const void* X, const void* W, const int32_t* labels, int64_t N,
                                int64_t H, int64_t V, fce_dtype dtype, const fce_options* opt,
                                float* loss, float* dX, float* dW, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return fused_impl(X, W, labels, N, H, V, dtype, opt, true, loss, dX, dW, workspace,
                    workspace_bytes, stream);
}

size_t fce_ce_logits_workspace_size(int64_t N) {
  if (N < 0) return 0;
  return fce::ce_workspace_bytes(N);
}

fce_status fce_ce_logits(const void* Z, int64_t ldz, const int32_t* labels, int64_t N, int64_t V,
                         fce_dtype dtype, const fce_options* opt, float* loss, float* lse,
                         void* dZ, int64_t lddz, const float* grad_loss, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (N < 0 || V < 1 || N >= (int64_t{1} << 31) || V >= (int64_t{1} << 30)) return FCE_ERR_SHAPE;
  if (workspace == nullptr) return FCE_ERR_NULL;
  if (N > 0 && (Z == nullptr || labels == nullptr || lse == nullptr)) return FCE_ERR_NULL;
  if (dtype != FCE_F32 && dtype != FCE_BF16) return FCE_ERR_ARG;
  fce::LossOpts lo;
  if (fce_status s = check_options(opt, true, kRecomputeOnly, &lo); s != FCE_OK) return s;
  const bool none = lo.reduction == fce::Reduction::None;
  if (loss == nullptr && !(none && N == 0)) return FCE_ERR_NULL;
  const int64_t es = (dtype == FCE_BF16) ? 2 : 4;
  // the kernel addresses a row with 32-bit byte offsets
  if (V * es >= (int64_t{1} << 31)) return FCE_ERR_SHAPE;
  if (ldz < V || (dZ != nullptr && lddz < V)) return FCE_ERR_SHAPE;
  if (dZ == Z && lddz != ldz) return FCE_ERR_ARG;
  if ((ldz * es) % 16 != 0 || (dZ != nullptr && (lddz * es) % 16 != 0)) return FCE_ERR_ALIGN;
  if ((N > 0 && !aligned16(Z)) || (dZ != nullptr && !aligned16(dZ)) || !aligned16(workspace))
    return FCE_ERR_ALIGN;
  if (workspace_bytes < fce::ce_workspace_bytes(N)) return FCE_ERR_WORKSPACE;
  if (fce_status s = check_device(); s != FCE_OK) return s;
  fce::CeLogitsCall c;
  c.Z = Z;
  c.ldz = ldz;
  c.dZ = dZ;
  c.lddz = dZ ? lddz : 0;
  c.labels = labels;
  c.N = N;
  c.V = V;
  c.bf16 = dtype == FCE_BF16;
  c.o = lo;
  c.grad = grad_loss;
  c.loss = loss;
  c.lse = lse;
  c.ws = static_cast<char*>(workspace);
  TimerScope ts;
  return from_hip(fce::launch_ce_logits(c, stream, ts.next()));
}

fce_status fce_fused_fwd_bwd_noalloc(const void* X, const void* W, const int32_t* labels,
                                     int64_t N, int64_t H, int64_t V, fce_dtype dtype,
                                     const fce_options* opt, float* loss, float* dX, float* dW,
                                     hipStream_t stream) {
  // the plan's workspace must fit the static scratch (checked before any
  // device call, like every other argument error)
  if (dtype != FCE_F32 && dtype != FCE_BF16) return FCE_ERR_ARG;
  const size_t need = fce_workspace_size_ex(N, H, V, dtype, opt);
  if (need == 0) {
    // invalid arguments: let the shared validation name them
    Plan p;
    fce::LossOpts lo;
    const fce_status s = validate(X, W, labels, N, H, V, dtype, opt, true, kAllVariants,
                                  FCE_STATIC_SCRATCH_BYTES, W, &p, &lo);
    return s != FCE_OK ? s : FCE_ERR_ARG;
  }
  if (need > FCE_STATIC_SCRATCH_BYTES) return FCE_ERR_WORKSPACE;
  if (fce_status s = check_device(); s != FCE_OK) return s;
  void* ws = nullptr;
  size_t bytes = 0;
  if (hipError_t e = fce::static_scratch(&ws, &bytes); e != hipSuccess) return from_hip(e);
  return fused_impl(X, W, labels, N, H, V, dtype, opt, true, loss, dX, dW, ws, bytes, stream);
}

fce_status fce_scale_grads(float* dX, int64_t n_dx, float* dW, int64_t n_dw,
                           const float* grad_loss, hipStream_t stream) {
  if (n_dx < 0 || n_dw < 0) return FCE_ERR_SHAPE;
  if (grad_loss == nullptr || (n_dx > 0 && dX == nullptr) || (n_dw > 0 && dW == nullptr))
    return FCE_ERR_NULL;
  if ((n_dx > 0 && !aligned16(dX)) || (n_dw > 0 && !aligned16(dW))) return FCE_ERR_ALIGN;
  if (n_dx == 0 && n_dw == 0) return FCE_OK;
  if (fce_status s = check_device(); s != FCE_OK) return s;
  TimerScope ts;
  return from_hip(fce::launch_scale_grads(dX, n_dx, dW, n_dw, grad_loss, stream, ts.next()));
}

fce_status fce_get_label_errors(const void* workspace, int32_t* host_count, hipStream_t stream) {
  if (workspace == nullptr || host_count == nullptr) return FCE_ERR_NULL;
  const fce::Ctrl* ctrl = static_cast<const fce::Ctrl*>(workspace);
  fce::Ctrl h;
  if (hipError_t e = hipMemcpyAsync(&h, ctrl, sizeof(h), hipMemcpyDeviceToHost, stream);
      e != hipSuccess)
    return from_hip(e);
  if (hipError_t e = hipStreamSynchronize(stream); e != hipSuccess) return from_hip(e);
  *host_count = h.n_invalid;
  return FCE_OK;
}

fce_status fce_get_filter_stats(const void* workspace, int64_t* kept_tiles, int64_t* all_tiles,
                                hipStream_t stream) {
  if (workspace == nullptr || kept_tiles == nullptr || all_tiles == nullptr) return FCE_ERR_NULL;
  unsigned long long h[2] = {0, 0};
  const char* src = static_cast<const char*>(workspace) + fce::kOffFilterStats;
  if (hipError_t e = hipMemcpyAsync(h, src, sizeof(h), hipMemcpyDeviceToHost, stream);
      e != hipSuccess)
    return from_hip(e);
  if (hipError_t e = hipStreamSynchronize(stream); e != hipSuccess) return from_hip(e);
  *kept_tiles = static_cast<int64_t>(h[0]);
  *all_tiles = static_cast<int64_t>(h[1]);
  return FCE_OK;
}

const char* fce_status_string(fce_status status) {
  switch (status) {
    case FCE_OK: return "ok";
    case FCE_ERR_NULL: return "a required pointer is NULL";
    case FCE_ERR_SHAPE: return "invalid shape (need N >= 0, H >= 1, V >= 1, extents < 2^30)";
    case FCE_ERR_ARG: return "invalid argument (dtype, reduction, schedule, chunk >= 1, 0 <= label_smoothing < 1)";
    case FCE_ERR_WORKSPACE: return "workspace smaller than fce_workspace_size()";
    case FCE_ERR_ALIGN: return "pointers must be 16-byte aligned and H a multiple of 8 (bf16) or 4 (fp32)";
    case FCE_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
    case FCE_ERR_HIP: return "HIP runtime error or kernel launch failure";
  }
  return "unknown status";
}

const char* fce_last_hip_error(void) {
  return t_last_hip == hipSuccess ? "none" : hipGetErrorString(t_last_hip);
}

fce_status fce_timing_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_timer_mu);
  if (enable) {
    // create the events now: creating them inside the timed calls can stall
    // the enqueueing thread long enough to leave the GPU idle
    while (g_timer.pool.size() < kTimerPreallocEvents) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return FCE_ERR_HIP;
      g_timer.pool.push_back(e);
    }
  }
  g_timer.enabled = enable != 0;
  g_timing_on.store(g_timer.enabled, std::memory_order_release);
  if (!g_timer.enabled) {
    g_timer.records.clear();
    g_timer.open = -1;
  }
  return FCE_OK;
}

fce_status fce_timing_read(fce_kernel_timing* out, int cap, int* count) {
  if (count == nullptr || (cap > 0 && out == nullptr)) return FCE_ERR_NULL;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  std::vector<fce_kernel_timing> agg;
  bool failed = g_timer.failed;
  for (const Record& r : g_timer.records) {
    float ms = 0.0f;
    if (r.stop < 0 || hipEventSynchronize(g_timer.pool[r.stop]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.pool[r.start], g_timer.pool[r.stop]) != hipSuccess) {
      failed = true;
      continue;
    }
    fce_kernel_timing* slot = nullptr;
    for (auto& a : agg)
      if (r.name == a.name) slot = &a;
    if (slot == nullptr) {
      fce_kernel_timing t;
      std::memset(&t, 0, sizeof(t));
      std::strncpy(t.name, r.name.c_str(), sizeof(t.name) - 1);
      agg.push_back(t);
      slot = &agg.back();
    }
    slot->launches += 1;
    slot->total_ms += ms;
    slot->flops += r.flops;
  }
  g_timer.records.clear();
  g_timer.used = 0;
  g_timer.open = -1;
  g_timer.last_stop = -1;
  g_timer.failed = false;
  const int n = static_cast<int>(agg.size());
  for (int i = 0; i < n && i < cap; ++i) out[i] = agg[i];
  *count = n;
  return failed ? FCE_ERR_HIP : FCE_OK;
}

}  // extern "C"
