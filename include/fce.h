/*
 * fce.h -- fused linear cross-entropy for AMD MI355X (gfx950): C ABI.
 *
 * The operation is the language-model-head loss over a vocabulary of V
 * classes.  With hidden states X[N,H], unembedding weights W[V,H] and labels
 * y[N]:
 *
 *   Z = X W^T                                  ("Chunked and Fused Cross-Entropy: How Online
 *                                                Logit Tiling Slashes ... VRAM Bottlenecks",
 *                                                llms.blog, "The Vocabulary Memory Wall")
 *   LSE_i = m_i + log sum_j exp(z_ij - m_i)      (same page, "Mathematical Mechanics", step 2)
 *   l_i   = LSE_i - (1-eps) z_{i,y_i} - (eps/V) sum_j z_ij      (eps = label_smoothing)
 *   loss  = sum_{i valid} l_i / D,  D = max(N_valid, 1) for mean, 1 for sum
 *   dZ_ij = (softmax_ij - (1-eps)[j = y_i] - eps/V) * g / D     (same page, step 3;
 *                                                "Fused cross-entropy -- the memory kernel",
 *                                                "The gradient that makes fusion trivial")
 *   dX = dZ W,  dW = dZ^T X                      (llms.blog step 4; lesson 27 "Trick 2")
 *
 * Rows whose label equals ignore_index carry no loss and no gradient
 * (llms.blog, "Numerical Considerations", item 2).  The N x V logits never
 * exist in device memory: the forward reduces each logit tile on chip with
 * the running max / sum-exp recurrence (lesson 27, "Trick 1"), and the
 * backward recomputes logit tiles into a scratch block of at most
 * chunk x V elements (llms.blog, "Mathematical Mechanics", step 1 and
 * "Peak Logit Memory Complexity"; lesson 27, "Worked number").
 *
 * Conventions shared by every entry point
 *   - Pointers named X, W, labels, loss, lse, grad_loss, dX, dW and the
 *     workspace are DEVICE pointers; every other argument is a host value.
 *   - X is row-major [N][H], W row-major [V][H]; both have the dtype given by
 *     `dtype` (FCE_BF16 or FCE_F32).  labels is int32[N], 0-based.
 *   - Outputs (loss, lse, dX, dW) are float32.  dX [N][H] and dW [V][H] are
 *     overwritten, never accumulated into.
 *   - The caller owns every buffer, including the workspace, whose size is
 *     given by fce_workspace_size().  The library never allocates or frees
 *     device memory and never synchronises the stream (except
 *     fce_get_label_errors and fce_timing_read, which say so).
 *   - Work is enqueued asynchronously on `stream`.  Calls sharing one
 *     workspace must be ordered on one stream.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs on the same device and build (no floating-point atomics).
 *   - Host-detectable argument errors return a negative status with nothing
 *     enqueued.  A label outside [0, V) that is not ignore_index is detected
 *     on the device: it is counted (fce_get_label_errors), its row is
 *     treated as ignored, and the loss is set to NaN.
 *   - Alignment: X, W, dX, dW and the workspace must be 16-byte aligned and
 *     H must be a multiple of 8 (bf16) or 4 (fp32), so that every row starts
 *     on a 16-byte boundary.
 *   - Shapes: N >= 0, H >= 1, V >= 1.  N = 0 gives loss 0 and dW = 0.
 *   - fce_forward, fce_backward and fce_fused_fwd_bwd take reduction
 *     FCE_MEAN or FCE_SUM (FCE_NONE is FCE_ERR_ARG there; see the *_ex
 *     entry points further down for it and for z-loss).
 *
 * `chunk` bounds the logit-space scratch of the backward pass to chunk x V
 * elements (bf16 for FCE_BF16, fp32 for FCE_F32, each dimension rounded up
 * to the kernel tile).  `schedule` chooses the shape of that block:
 *   FCE_SCHED_TOKEN  chunk tokens x all V, as the pages describe;
 *   FCE_SCHED_VOCAB  all N tokens x (chunk*V/N) vocabulary columns;
 *   FCE_SCHED_AUTO   the block shape with the same budget that moves the
 *                    fewest fp32 gradient bytes (see fce_plan).
 * The loss and gradients are the same up to fp32 summation order.
 *
 * Plans are cached by (N, H, V, dtype, chunk, schedule, variant): the first
 * call with a key runs the block-shape search on the host (milliseconds,
 * tens of them at the largest shapes), later calls reuse its result.  The
 * cache is process-wide, guarded by a mutex, and holds up to 256 plans.
 */
#ifndef FCE_H
#define FCE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FCE_OK = 0,
  FCE_ERR_NULL = -1,      /* a required pointer is NULL */
  FCE_ERR_SHAPE = -2,     /* N < 0, H < 1, V < 1, N >= 2^30, or H or V near or above
                             2^22 (bf16) / 2^21 (fp32): 256 rows of H or V elements
                             must stay under 2 GiB */
  FCE_ERR_ARG = -3,       /* bad enum or option, chunk < 1, label_smoothing outside [0,1) */
  FCE_ERR_WORKSPACE = -4, /* workspace smaller than fce_workspace_size() */
  FCE_ERR_ALIGN = -5,     /* pointer not 16-byte aligned or H not a multiple of 8 / 4 */
  FCE_ERR_DEVICE = -6,    /* current device is not gfx950 */
  FCE_ERR_HIP = -7        /* a HIP runtime call or kernel launch failed */
} fce_status;

typedef enum { FCE_F32 = 0, FCE_BF16 = 1 } fce_dtype;
/* FCE_NONE (per-token losses) is accepted by the *_ex entry points only. */
typedef enum { FCE_MEAN = 0, FCE_SUM = 1, FCE_NONE = 2 } fce_reduction;
typedef enum { FCE_SCHED_AUTO = 0, FCE_SCHED_TOKEN = 1, FCE_SCHED_VOCAB = 2 } fce_schedule;
/* How the backward gets its logits (fce_options.variant).
 * FCE_VARIANT_RECOMPUTE: rebuild each logit block from X and W (8NVH FLOPs
 *   per forward + backward; lesson 27, "Trick 2").  With FCE_BF16 the
 *   workspace also holds X^T, H x (N rounded up to 256) bf16, written once
 *   per backward for the dW products.
 * FCE_VARIANT_STORE_LOGITS: fce_fused_fwd_bwd_ex only.  The forward keeps each
 *   chunk's logits, [C][V rounded up to the tile] in the dtype of X, in the
 *   workspace, and the backward overwrites them in place with dZ (6NVH FLOPs;
 *   llms.blog, "LinkedIn Liger Kernel").  C is `chunk` rounded up to 256
 *   tokens; the logit buffer is C x V elements, and dW is re-read once per
 *   chunk after the first.
 * FCE_VARIANT_FILTERED: FCE_BF16 only; the *_ex forward, backward, fused and
 *   workspace calls.  RECOMPUTE with gradient filtering (llms.blog, "Apple Cut
 *   Cross-Entropy (CCE)"): a 256 x 256 tile of dZ (tokens x vocabulary) in
 *   which every softmax value is below 2^-12 and no token's label falls is
 *   treated as zero and left out of dX and dW.  An approximation: dropped
 *   entries are each below 2^-12 in magnitude (before the g/D scale); the loss
 *   and LSE are exact as in RECOMPUTE.  fce_get_filter_stats reports how many
 *   tiles were kept. */
typedef enum {
  FCE_VARIANT_RECOMPUTE = 0,
  FCE_VARIANT_STORE_LOGITS = 1,
  FCE_VARIANT_FILTERED = 2
} fce_variant;

/* The backward schedule chosen for a problem (host-only, no GPU needed). */
typedef struct {
  int64_t block_tokens;     /* tokens per logit block (C_N)                        */
  int64_t block_vocab;      /* vocabulary columns per logit block (C_V)            */
  int64_t n_token_blocks;   /* ceil(N / C_N)                                       */
  int64_t n_vocab_blocks;   /* ceil(V / C_V)                                       */
  int64_t scratch_bytes;    /* logit-space device bytes: the dZ block, tile-padded */
  int64_t partial_bytes;    /* forward per-(split, token) LSE partials             */
  int64_t workspace_bytes;  /* == fce_workspace_size()                             */
  int64_t fwd_splits;       /* vocabulary splits of the forward reduction          */
  int64_t grad_rmw_bytes;   /* fp32 dX/dW bytes written + re-read across blocks    */
  int64_t dx_splits;        /* splits of the dX product over V (fp32 partials)     */
} fce_plan_info;

/* Loss options of the *_ex entry points.  Fields are fixed-width so the
 * layout is the same for every caller (32 bytes). */
typedef struct {
  int32_t ignore_index;   /* a label equal to this carries no loss (usually -100)        */
  float label_smoothing;  /* eps in [0, 1)                                               */
  float z_loss;           /* alpha >= 0, finite: adds alpha * LSE_i^2 to each valid row's
                             loss (llms.blog, "Numerical Considerations", item 3)       */
  int32_t reduction;      /* fce_reduction: FCE_MEAN, FCE_SUM or FCE_NONE               */
  int64_t chunk;          /* logit-space budget, chunk x V elements (>= 1)              */
  int32_t schedule;       /* fce_schedule                                               */
  int32_t variant;        /* fce_variant; FCE_VARIANT_STORE_LOGITS only where stated    */
} fce_options;

/* Size in bytes of the workspace the three compute entry points need for
 * this problem (host-only).  Returns 0 if the arguments are invalid. */
size_t fce_workspace_size(int64_t N, int64_t H, int64_t V, fce_dtype dtype, int64_t chunk,
                          fce_schedule schedule);

/* Fill *out with the plan the compute entry points will use (host-only). */
fce_status fce_plan(int64_t N, int64_t H, int64_t V, fce_dtype dtype, int64_t chunk,
                    fce_schedule schedule, fce_plan_info* out);

/* Forward pass (llms.blog "Mathematical Mechanics" steps 1-2; aifetchly
 * "Cut Cross-Entropy ... Guide", "Online Log-Sum-Exp Accumulation").
 * Writes loss[1] (device) and lse[N] (device; LSE of every valid row, NaN
 * on ignored rows), which fce_backward needs. */
fce_status fce_forward(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                       int64_t V, fce_dtype dtype, int32_t ignore_index, float label_smoothing,
                       fce_reduction reduction, int64_t chunk, fce_schedule schedule, float* loss,
                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward pass with recomputation (lesson 27 "Trick 1": the gradient tile
 * is rebuilt from the saved LSE; "Trick 2": it feeds dX = dZ W and
 * dW += dZ^T X block by block).  lse[N] must come from fce_forward with the
 * same inputs.  grad_loss is a device pointer to the upstream scalar
 * gradient g, or NULL for g = 1.  Overwrites dX[N][H] and dW[V][H]. */
fce_status fce_backward(const void* X, const void* W, const int32_t* labels, int64_t N, int64_t H,
                        int64_t V, fce_dtype dtype, int32_t ignore_index, float label_smoothing,
                        fce_reduction reduction, int64_t chunk, fce_schedule schedule,
                        const float* lse, const float* grad_loss, float* dX, float* dW,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward then backward with g = 1 in one call; the LSE stays in the
 * workspace.  With FCE_BF16, bitwise identical to fce_forward followed by
 * fce_backward.  With FCE_F32 the backward takes its exponents from the
 * forward's split row statistics (row max m and log2 of the sum of
 * exp(z - m), kept in the workspace) as (z - m) log2e - log2 l, exact near
 * the max at any |LSE|; the split calls pass the LSE as one rounded fp32
 * value per row instead, which puts a relative error of up to |LSE| 2^-25
 * on every softmax value of the row, so the two agree to that rounding
 * ("Cut Cross-Entropy ... Guide", "Numerical Stability and Maximum
 * Subtraction on Chip": subtract the row maximum before exponentiating). */
fce_status fce_fused_fwd_bwd(const void* X, const void* W, const int32_t* labels, int64_t N,
                             int64_t H, int64_t V, fce_dtype dtype, int32_t ignore_index,
                             float label_smoothing, fce_reduction reduction, int64_t chunk,
                             fce_schedule schedule, float* loss, float* dX, float* dW,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- The entry point that allocates nothing.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * fce_fused_fwd_bwd_ex with the library's own static scratch as the
 * workspace.  The scratch is a device array of FCE_STATIC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends (one copy per
 * GPU); the call itself allocates nothing.  The caller still passes inputs
 * and outputs, as for fce_fused_fwd_bwd_ex, whose arguments, options and
 * results this call shares bitwise.  A problem whose workspace
 * (fce_workspace_size_ex with the same options) exceeds
 * FCE_STATIC_SCRATCH_BYTES returns FCE_ERR_WORKSPACE with nothing enqueued;
 * a smaller chunk, or FCE_SCHED_TOKEN, shrinks the workspace.  Every call
 * on one GPU uses that GPU's one scratch: calls that overlap on one GPU
 * (different streams, or threads without ordering) race and must not be
 * made; calls ordered on one stream are safe.  The scratch keeps the last
 * call's contents; nothing in it needs to start at zero, since each call
 * writes every byte of it that it reads. */
#define FCE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

fce_status fce_fused_fwd_bwd_noalloc(const void* X, const void* W, const int32_t* labels,
                                     int64_t N, int64_t H, int64_t V, fce_dtype dtype,
                                     const fce_options* opt, float* loss, float* dX, float* dW,
                                     hipStream_t stream);

/* Applies the upstream scalar gradient to gradients computed with g = 1:
 * dX[i] *= g for i < n_dx and dW[j] *= g for j < n_dw, in place, where g is
 * the device scalar grad_loss[0] (chain rule of the loss scale; llms.blog,
 * "Mathematical Mechanics", step 3, with the upstream gradient of an
 * autograd backward).  For the store-logits variant, whose fused call
 * computes dX and dW in the forward pass of a training step, before the
 * upstream gradient exists ("LinkedIn Liger Kernel").  All pointers DEVICE;
 * dX and dW 16-byte aligned when their count is positive.  Errors:
 * FCE_ERR_SHAPE for a negative count, FCE_ERR_NULL for grad_loss or a
 * needed array NULL, FCE_ERR_ALIGN, FCE_ERR_DEVICE; nothing is enqueued
 * then.  Enqueued on `stream`, no synchronisation. */
fce_status fce_scale_grads(float* dX, int64_t n_dx, float* dW, int64_t n_dw,
                           const float* grad_loss, hipStream_t stream);

/* Number of labels outside [0, V) that were not ignore_index in the last
 * call that used this workspace.  Synchronises `stream`. */
fce_status fce_get_label_errors(const void* workspace, int32_t* host_count, hipStream_t stream);

/* dZ tiles kept and tiles in all by the last backward with
 * FCE_VARIANT_FILTERED that used this workspace (host outputs; token blocks
 * whose labels are all ignored are counted as skipped).  Undefined after
 * other calls.  Synchronises `stream`. */
fce_status fce_get_filter_stats(const void* workspace, int64_t* kept_tiles, int64_t* all_tiles,
                                hipStream_t stream);

/* ---- Entry points with loss options (fce_options).
 *
 * The same operation as fce_forward / fce_backward / fce_fused_fwd_bwd, with
 * two more loss terms and one more reduction:
 *   l_i  = LSE_i - (1-eps) z_{i,y_i} - (eps/V) sum_j z_ij + alpha LSE_i^2
 *   dZ_ij = (softmax_ij (1 + 2 alpha LSE_i) - (1-eps)[j = y_i] - eps/V) * s_i
 * with s_i = g / D for FCE_MEAN and FCE_SUM (g the scalar upstream
 * gradient), and s_i = g_i for FCE_NONE (one upstream gradient per token).
 * For FCE_NONE the loss output is float[N]: l_i for a valid row, 0 for an
 * ignored row, NaN for a label outside [0, V) that is not ignore_index.
 * `opt` is a host pointer; NULL is FCE_ERR_NULL.  A z_loss that is negative,
 * infinite or NaN, an unknown reduction, schedule or variant, chunk < 1,
 * FCE_VARIANT_STORE_LOGITS anywhere but fce_fused_fwd_bwd_ex and
 * fce_workspace_size_ex, or FCE_VARIANT_FILTERED with FCE_F32 is FCE_ERR_ARG
 * (the size query returns 0).  With the default-valued options
 * (z_loss 0, reduction mean or sum) they equal the entry points above
 * bitwise.  Everything else is as documented above. */

/* Workspace size for these options (host-only; 0 if arguments are invalid). */
size_t fce_workspace_size_ex(int64_t N, int64_t H, int64_t V, fce_dtype dtype,
                             const fce_options* opt);

/* Forward: loss (float[1], or float[N] for FCE_NONE) and lse[N]. */
fce_status fce_forward_ex(const void* X, const void* W, const int32_t* labels, int64_t N,
                          int64_t H, int64_t V, fce_dtype dtype, const fce_options* opt,
                          float* loss, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Backward: grad_loss is float[1] (FCE_MEAN, FCE_SUM) or float[N]
 * (FCE_NONE), device, or NULL for ones.  lse from fce_forward_ex with the
 * same X, W, labels and options. */
fce_status fce_backward_ex(const void* X, const void* W, const int32_t* labels, int64_t N,
                           int64_t H, int64_t V, fce_dtype dtype, const fce_options* opt,
                           const float* lse, const float* grad_loss, float* dX, float* dW,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Fused forward and backward with upstream gradient 1 (for FCE_NONE: 1 for
 * every token).  With opt->variant = FCE_VARIANT_STORE_LOGITS the logits are
 * kept per chunk instead of recomputed (schedule is then unused); the
 * workspace must be sized by fce_workspace_size_ex with the same options. */
fce_status fce_fused_fwd_bwd_ex(const void* X, const void* W, const int32_t* labels, int64_t N,
                                int64_t H, int64_t V, fce_dtype dtype, const fce_options* opt,
                                float* loss, float* dX, float* dW, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---- Loss on logits the caller holds ("Fused cross-entropy -- the memory
 * kernel", lesson 27: "Trick 1" alone, the logit-space memory table's fused
 * softmax+CE row, where probs and dlogits reuse the logits buffer).
 *
 * Z is DEVICE, row-major [N][ldz] with ldz >= V (elements), dtype FCE_BF16
 * or FCE_F32, 16-byte aligned with ldz * element size a multiple of 16.  A
 * row of V elements must be under 2 GiB (FCE_ERR_SHAPE otherwise).
 * Writes lse[N] and the loss (float[1], or float[N] for FCE_NONE) as in
 * fce_forward_ex.  If dZ is not NULL it also writes
 *   dZ_ij = (softmax_ij (1 + 2 alpha LSE_i) - (1-eps)[j = y_i] - eps/V) * s_i
 * (s_i as in fce_backward_ex, from grad_loss: float[1] or float[N], or NULL
 * for ones) in Z's dtype, row-major [N][lddz]; dZ may be Z itself (the
 * gradient then overwrites the logits; lddz must equal ldz).  Columns
 * V .. of a row's last 16-byte vector are written as 0 in dZ; columns
 * past that are not touched.  Ignored rows get dZ = 0.  opt->chunk and
 * opt->schedule are checked as elsewhere but unused; opt->variant must be
 * FCE_VARIANT_RECOMPUTE.
 * The workspace (fce_ce_logits_workspace_size) holds the label scan and
 * per-row loss terms. */
size_t fce_ce_logits_workspace_size(int64_t N);

fce_status fce_ce_logits(const void* Z, int64_t ldz, const int32_t* labels, int64_t N, int64_t V,
                         fce_dtype dtype, const fce_options* opt, float* loss, float* lse,
                         void* dZ, int64_t lddz, const float* grad_loss, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* fce_status_string(fce_status status);

/* The HIP runtime's description of the last HIP error behind an
 * FCE_ERR_HIP returned to the calling thread, or "none".  The string is
 * static (owned by the HIP runtime); the record is per thread and is
 * overwritten by the next such error. */
const char* fce_last_hip_error(void);

/* Per-kernel timing.  While enabled, every kernel the library launches is
 * bracketed by HIP events on the caller's stream; within one call,
 * consecutive kernels share the event between them (one event per kernel
 * boundary), and each call starts with an event of its own, so work the
 * caller enqueues between calls is never counted.  The events cost the
 * stream a few microseconds each.  fce_timing_enable(1) creates a pool of
 * events first (more are created only when a run of calls between reads
 * needs them), and returns FCE_ERR_HIP if it cannot.  fce_timing_read synchronises on the
 * recorded events, fills up to `cap` entries and resets the counters.  The
 * timer is process-wide and guarded by a mutex: while it is enabled, each
 * entry point holds that mutex while it enqueues its launches, so calls
 * from several threads are serialised and their records do not interleave;
 * while it is disabled no lock is taken. */
typedef struct {
  char name[32];        /* kernel family: "fwd_lse", "bwd_dz", "bwd_dw", "bwd_dx", ... */
  int64_t launches;     /* launches recorded                                      */
  double total_ms;      /* summed event-to-event time                             */
  double flops;         /* algorithmic flops of those launches (0 if not a GEMM)  */
} fce_kernel_timing;

fce_status fce_timing_enable(int enable);
fce_status fce_timing_read(fce_kernel_timing* out, int cap, int* count);

#ifdef __cplusplus
}
#endif

#endif /* FCE_H */
