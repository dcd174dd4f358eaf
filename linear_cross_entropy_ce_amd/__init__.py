"""Fused linear cross-entropy for AMD MI355X (gfx950).

The computation runs entirely in the HIP library ``lib/libfce.so`` (C ABI in
``include/fce.h``).  This package only marshals arguments: torch provides
device memory and the stream.

    loss = linear_cross_entropy(hidden, weight, labels, ignore_index=-100)
    loss.backward()

No N x V logits tensor is ever allocated: the forward reduces logit tiles on
chip, the backward recomputes them into a scratch block of at most
chunk x V elements ("Chunked and Fused Cross-Entropy", llms.blog,
"Mathematical Mechanics"; "Fused cross-entropy -- the memory kernel",
"Trick 2").
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    FCE_BF16,
    FCE_F32,
    FceError,
    SCHEDULES,
    FCE_NONE,
    FCE_VARIANT_RECOMPUTE,
    FCE_VARIANT_STORE_LOGITS,
    FCE_VARIANT_FILTERED,
    REDUCTIONS,
    VARIANTS,
    fce_backward,
    fce_backward_ex,
    fce_ce_logits,
    fce_ce_logits_workspace_size,
    fce_forward,
    fce_forward_ex,
    fce_fused_fwd_bwd,
    fce_fused_fwd_bwd_ex,
    fce_fused_fwd_bwd_noalloc,
    STATIC_SCRATCH_BYTES,
    fce_workspace_size_ex,
    make_options,
    fce_get_label_errors,
    fce_get_filter_stats,
    fce_plan,
    fce_scale_grads,
    status_string,
    fce_timing_enable,
    fce_timing_read,
    fce_workspace_size,
    load_library,
)
from .memory import logit_space_bytes  # noqa: F401


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return FCE_BF16
    if t.dtype == torch.float32:
        return FCE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def workspace_for(N, H, V, dtype, chunk=1024, schedule="auto", device="cuda", **options):
    """A uint8 workspace tensor of the size the library asks for (``options``:
    those of the *_ex entry points, e.g. ``variant="store_logits"``)."""
    import torch

    code = dtype if isinstance(dtype, int) else (FCE_BF16 if dtype == torch.bfloat16 else FCE_F32)
    if options:
        n = fce_workspace_size_ex(N, H, V, code, chunk=chunk, schedule=schedule, **options)
    else:
        n = fce_workspace_size(N, H, V, code, chunk, SCHEDULES.get(schedule, schedule))
    if n == 0:
        raise ValueError("invalid problem for fce_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _make_function():
    import torch

    class _LinearCrossEntropy(torch.autograd.Function):
        @staticmethod
        def forward(ctx, hidden, weight, labels, opts):
            H = hidden.shape[-1]
            X = hidden.reshape(-1, H).contiguous()
            W = weight.contiguous()
            if X.dtype != W.dtype:
                raise TypeError("hidden and weight must share a dtype")
            y = labels.reshape(-1).to(torch.int32).contiguous()
            N, V = X.shape[0], W.shape[0]
            code = FCE_BF16 if X.dtype == torch.bfloat16 else FCE_F32
            n = fce_workspace_size_ex(N, H, V, code, **opts)
            if n == 0:
                raise ValueError("invalid problem or options for fce_workspace_size_ex")
            ws = torch.empty(n, dtype=torch.uint8, device=X.device)
            none = opts["reduction"] == "none"
            loss = torch.empty(N if none else 1, dtype=torch.float32, device=X.device)
            ctx.cfg = (opts, hidden.shape, hidden.dtype, weight.dtype)
            if opts["variant"] == "store_logits":
                # gradients with an upstream gradient of 1, computed now; the
                # backward has the library scale them by the scalar it
                # receives (once: they are freed there, as autograd frees
                # saved buffers after a backward)
                dX = torch.empty((N, H), dtype=torch.float32, device=X.device)
                dW = torch.empty(W.shape, dtype=torch.float32, device=X.device)
                fce_fused_fwd_bwd_ex(X if N else None, W, y if N else None, loss,
                                     dX if N else None, dW, ws, **opts)
                ctx.grads = (dX, dW)
                return loss[0]
            lse = torch.empty(max(N, 1), dtype=torch.float32, device=X.device)
            fce_forward_ex(X if N else None, W, y if N else None, loss if loss.numel() else None,
                           lse, ws, **opts)
            ctx.save_for_backward(X, W, y, lse)
            ctx.ws = ws
            return loss.reshape(labels.shape) if none else loss[0]

        @staticmethod
        def backward(ctx, g):
            opts, hshape, hdt, wdt = ctx.cfg
            if opts["variant"] == "store_logits":
                if ctx.grads is None:
                    raise RuntimeError("the store_logits variant keeps its gradients for one "
                                       "backward pass only")
                dX, dW = ctx.grads
                ctx.grads = None
                g1 = g.reshape(1).to(torch.float32).contiguous()
                fce_scale_grads(dX if dX.numel() else None, dW, g1)
                return dX.to(hdt).reshape(hshape), dW.to(wdt), None, None
            X, W, y, lse = ctx.saved_tensors
            N, H = X.shape
            g1 = g.reshape(-1).to(torch.float32).contiguous()
            dX = torch.empty((N, H), dtype=torch.float32, device=X.device)
            dW = torch.empty(W.shape, dtype=torch.float32, device=X.device)
            fce_backward_ex(X if N else None, W, y if N else None, lse,
                            g1 if g1.numel() else None, dX if N else None, dW, ctx.ws, **opts)
            return dX.to(hdt).reshape(hshape), dW.to(wdt), None, None

    return _LinearCrossEntropy


_FN = None


def linear_cross_entropy(hidden, weight, labels, ignore_index: int = -100,
                         label_smoothing: float = 0.0, reduction: str = "mean", chunk: int = 1024,
                         schedule: str = "auto", z_loss: float = 0.0,
                         variant: str = "recompute"):
    """Cross-entropy of ``hidden @ weight.T`` against ``labels``: a scalar for
    reduction "mean" or "sum", per-token losses (labels' shape) for "none".

    hidden [..., H] and weight [V, H] share a dtype (bfloat16 or float32);
    labels [...] are class indices, ``ignore_index`` rows carry no loss.
    ``z_loss`` = alpha adds alpha * logsumexp(z)^2 per token.  Gradients for
    hidden and weight come from the fused backward.

    variant: "recompute" (the backward rebuilds the logits), "filtered"
    (bfloat16: the gradient filtering approximation, dZ tiles whose softmax
    values are all below 2^-12 skipped) or "store_logits" (mean or sum only:
    the forward computes the gradients too, keeping each chunk's logits, and
    holds dX and dW in fp32 until the backward, where the library scales
    them by the upstream gradient; one backward per forward)."""
    global _FN
    if _FN is None:
        _FN = _make_function()
    if reduction not in REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if variant == "store_logits" and reduction == "none":
        raise ValueError("variant 'store_logits' needs a scalar loss (reduction mean or sum)")
    opts = dict(ignore_index=ignore_index, label_smoothing=label_smoothing, z_loss=z_loss,
                reduction=reduction, chunk=chunk, schedule=schedule, variant=variant)
    return _FN.apply(hidden, weight, labels, opts)
