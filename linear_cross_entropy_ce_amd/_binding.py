"""ctypes binding of libfce.so: the C ABI's entry points under the same names.

Argument marshalling only.  Tensors are passed by device pointer, the
current torch stream is passed as the HIP stream, and every computation
runs in the library's HIP kernels.  Loading fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libfce.so")

FCE_OK = 0
FCE_ERR_NULL = -1
FCE_ERR_SHAPE = -2
FCE_ERR_ARG = -3
FCE_ERR_WORKSPACE = -4
FCE_ERR_ALIGN = -5
FCE_ERR_DEVICE = -6
FCE_ERR_HIP = -7

FCE_F32 = 0
FCE_BF16 = 1
FCE_MEAN = 0
FCE_SUM = 1
FCE_NONE = 2
SCHED_AUTO = 0
SCHED_TOKEN = 1
SCHED_VOCAB = 2
SCHEDULES = {"auto": SCHED_AUTO, "token": SCHED_TOKEN, "vocab": SCHED_VOCAB}
REDUCTIONS = {"mean": FCE_MEAN, "sum": FCE_SUM, "none": FCE_NONE}
FCE_VARIANT_RECOMPUTE, FCE_VARIANT_STORE_LOGITS, FCE_VARIANT_FILTERED = 0, 1, 2
VARIANTS = {"recompute": FCE_VARIANT_RECOMPUTE, "store_logits": FCE_VARIANT_STORE_LOGITS,
            "filtered": FCE_VARIANT_FILTERED}

EXPORTED = ("fce_workspace_size", "fce_plan", "fce_forward", "fce_backward", "fce_fused_fwd_bwd",
            "fce_workspace_size_ex", "fce_forward_ex", "fce_backward_ex", "fce_fused_fwd_bwd_ex",
            "fce_ce_logits_workspace_size", "fce_ce_logits",
            "fce_get_label_errors", "fce_get_filter_stats", "fce_status_string",
            "fce_last_hip_error",
            "fce_timing_enable", "fce_timing_read")


class FceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)} (status {status})"
        if status == FCE_ERR_HIP:
            msg += f": {load_library().fce_last_hip_error().decode()}"
        super().__init__(msg)


class PlanInfo(ctypes.Structure):
    _fields_ = [("block_tokens", ctypes.c_int64), ("block_vocab", ctypes.c_int64),
                ("n_token_blocks", ctypes.c_int64), ("n_vocab_blocks", ctypes.c_int64),
                ("scratch_bytes", ctypes.c_int64), ("partial_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("fwd_splits", ctypes.c_int64),
                ("grad_rmw_bytes", ctypes.c_int64), ("dx_splits", ctypes.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class Options(ctypes.Structure):
    """fce_options (include/fce.h)."""
    _fields_ = [("ignore_index", ctypes.c_int32), ("label_smoothing", ctypes.c_float),
                ("z_loss", ctypes.c_float), ("reduction", ctypes.c_int32),
                ("chunk", ctypes.c_int64), ("schedule", ctypes.c_int32),
                ("variant", ctypes.c_int32)]


def make_options(ignore_index=-100, label_smoothing=0.0, z_loss=0.0, reduction="mean", chunk=1024,
                 schedule="auto", variant=0) -> Options:
    return Options(int(ignore_index), float(label_smoothing), float(z_loss),
                   REDUCTIONS.get(reduction, reduction), int(chunk),
                   SCHEDULES.get(schedule, schedule), int(VARIANTS.get(variant, variant)))


class KernelTiming(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfce.so (built by ``python -m linear_cross_entropy_ce_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          f"`python -m linear_cross_entropy_ce_amd.build`")
    # torch wheels carry their own HIP runtime.  Load it first, so that
    # libfce.so binds to the same runtime that owns torch's memory and
    # streams instead of pulling in a second one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i64, u64, i32, f32, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    lib.fce_workspace_size.restype = u64
    lib.fce_workspace_size.argtypes = [i64, i64, i64, i32, i64, i32]
    lib.fce_plan.restype = i32
    lib.fce_plan.argtypes = [i64, i64, i64, i32, i64, i32, ctypes.POINTER(PlanInfo)]
    common = [vp, vp, vp, i64, i64, i64, i32, i32, f32, i32, i64, i32]
    lib.fce_forward.restype = i32
    lib.fce_forward.argtypes = common + [vp, vp, vp, u64, vp]
    lib.fce_backward.restype = i32
    lib.fce_backward.argtypes = common + [vp, vp, vp, vp, vp, u64, vp]
    lib.fce_fused_fwd_bwd.restype = i32
    lib.fce_fused_fwd_bwd.argtypes = common + [vp, vp, vp, vp, u64, vp]
    op = ctypes.POINTER(Options)
    lib.fce_workspace_size_ex.restype = u64
    lib.fce_workspace_size_ex.argtypes = [i64, i64, i64, i32, op]
    common_ex = [vp, vp, vp, i64, i64, i64, i32, op]
    lib.fce_forward_ex.restype = i32
    lib.fce_forward_ex.argtypes = common_ex + [vp, vp, vp, u64, vp]
    lib.fce_backward_ex.restype = i32
    lib.fce_backward_ex.argtypes = common_ex + [vp, vp, vp, vp, vp, u64, vp]
    lib.fce_fused_fwd_bwd_ex.restype = i32
    lib.fce_fused_fwd_bwd_ex.argtypes = common_ex + [vp, vp, vp, vp, u64, vp]
    lib.fce_ce_logits_workspace_size.restype = u64
    lib.fce_ce_logits_workspace_size.argtypes = [i64]
    lib.fce_ce_logits.restype = i32
    lib.fce_ce_logits.argtypes = [vp, i64, vp, i64, i64, i32, op, vp, vp, vp, i64, vp, vp, u64, vp]
    lib.fce_get_label_errors.restype = i32
    lib.fce_get_label_errors.argtypes = [vp, ctypes.POINTER(i32), vp]
    lib.fce_get_filter_stats.restype = i32
    lib.fce_get_filter_stats.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), vp]
    lib.fce_status_string.restype = ctypes.c_char_p
    lib.fce_status_string.argtypes = [i32]
    lib.fce_last_hip_error.restype = ctypes.c_char_p
    lib.fce_last_hip_error.argtypes = []
    lib.fce_timing_enable.restype = i32
    lib.fce_timing_enable.argtypes = [i32]
    lib.fce_timing_read.restype = i32
    lib.fce_timing_read.argtypes = [ctypes.POINTER(KernelTiming), i32, ctypes.POINTER(i32)]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fce_status_string(status).decode()


def _check(status: int, where: str):
    if status != FCE_OK:
        raise FceError(status, where)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return FCE_BF16
    if t.dtype == torch.float32:
        return FCE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def fce_workspace_size(N, H, V, dtype, chunk, schedule=SCHED_AUTO) -> int:
    return int(load_library().fce_workspace_size(N, H, V, dtype, chunk, schedule))


def fce_plan(N, H, V, dtype, chunk, schedule=SCHED_AUTO) -> dict:
    info = PlanInfo()
    _check(load_library().fce_plan(N, H, V, dtype, chunk, schedule, ctypes.byref(info)), "fce_plan")
    return info.as_dict()


def _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule):
    N, H = (X.shape[0], X.shape[1]) if X is not None else (0, W.shape[1])
    V = W.shape[0]
    return [_ptr(X), _ptr(W), _ptr(labels), N, H, V, _dtype_code(W), int(ignore_index),
            float(label_smoothing), REDUCTIONS.get(reduction, reduction), int(chunk),
            SCHEDULES.get(schedule, schedule)]


def fce_forward(X, W, labels, loss, lse, workspace, ignore_index=-100, label_smoothing=0.0,
                reduction="mean", chunk=1024, schedule="auto", stream=None):
    args = _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule)
    st = load_library().fce_forward(*args, _ptr(loss), _ptr(lse), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fce_forward")


def fce_backward(X, W, labels, lse, grad_loss, dX, dW, workspace, ignore_index=-100,
                 label_smoothing=0.0, reduction="mean", chunk=1024, schedule="auto", stream=None):
    args = _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule)
    st = load_library().fce_backward(*args, _ptr(lse), _ptr(grad_loss), _ptr(dX), _ptr(dW),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check(st, "fce_backward")


def fce_fused_fwd_bwd(X, W, labels, loss, dX, dW, workspace, ignore_index=-100,
                      label_smoothing=0.0, reduction="mean", chunk=1024, schedule="auto",
                      stream=None):
    args = _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule)
    st = load_library().fce_fused_fwd_bwd(*args, _ptr(loss), _ptr(dX), _ptr(dW), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream))
    _check(st, "fce_fused_fwd_bwd")


def fce_workspace_size_ex(N, H, V, dtype, **options) -> int:
    o = make_options(**options)
    return int(load_library().fce_workspace_size_ex(N, H, V, dtype, ctypes.byref(o)))


def _common_ex(X, W, labels):
    N, H = (X.shape[0], X.shape[1]) if X is not None else (0, W.shape[1])
    return [_ptr(X), _ptr(W), _ptr(labels), N, H, W.shape[0], _dtype_code(W)]


def _ws(workspace):
    return [_ptr(workspace), workspace.numel() * workspace.element_size()]


def fce_forward_ex(X, W, labels, loss, lse, workspace, stream=None, **options):
    o = make_options(**options)
    st = load_library().fce_forward_ex(*_common_ex(X, W, labels), ctypes.byref(o), _ptr(loss),
                                       _ptr(lse), *_ws(workspace), _stream(stream))
    _check(st, "fce_forward_ex")


def fce_backward_ex(X, W, labels, lse, grad_loss, dX, dW, workspace, stream=None, **options):
    o = make_options(**options)
    st = load_library().fce_backward_ex(*_common_ex(X, W, labels), ctypes.byref(o), _ptr(lse),
                                        _ptr(grad_loss), _ptr(dX), _ptr(dW), *_ws(workspace),
                                        _stream(stream))
    _check(st, "fce_backward_ex")


def fce_fused_fwd_bwd_ex(X, W, labels, loss, dX, dW, workspace, stream=None, **options):
    o = make_options(**options)
    st = load_library().fce_fused_fwd_bwd_ex(*_common_ex(X, W, labels), ctypes.byref(o),
                                             _ptr(loss), _ptr(dX), _ptr(dW), *_ws(workspace),
                                             _stream(stream))
    _check(st, "fce_fused_fwd_bwd_ex")


def fce_ce_logits_workspace_size(N) -> int:
    return int(load_library().fce_ce_logits_workspace_size(N))


def fce_ce_logits(Z, labels, loss, lse, workspace, dZ=None, grad_loss=None, V=None, stream=None,
                  **options):
    """Loss (and dZ, which may be Z) on given logits Z [N, ldz]; V defaults
    to Z's row length."""
    o = make_options(**options)
    N, ldz = Z.shape
    V = ldz if V is None else V
    lddz = dZ.shape[1] if dZ is not None else 0
    st = load_library().fce_ce_logits(_ptr(Z), ldz, _ptr(labels), N, V, _dtype_code(Z),
                                      ctypes.byref(o), _ptr(loss), _ptr(lse), _ptr(dZ), lddz,
                                      _ptr(grad_loss), *_ws(workspace), _stream(stream))
    _check(st, "fce_ce_logits")


def fce_get_label_errors(workspace, stream=None) -> int:
    n = ctypes.c_int32(0)
    _check(load_library().fce_get_label_errors(_ptr(workspace), ctypes.byref(n), _stream(stream)),
           "fce_get_label_errors")
    return int(n.value)


def fce_get_filter_stats(workspace, stream=None) -> tuple:
    """(kept, all) dZ tiles of the last filtered backward on this workspace."""
    kept, total = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(load_library().fce_get_filter_stats(_ptr(workspace), ctypes.byref(kept),
                                               ctypes.byref(total), _stream(stream)),
           "fce_get_filter_stats")
    return int(kept.value), int(total.value)


def fce_timing_enable(enable: bool):
    _check(load_library().fce_timing_enable(1 if enable else 0), "fce_timing_enable")


def fce_timing_read() -> dict:
    cap = 32
    arr = (KernelTiming * cap)()
    n = ctypes.c_int32(0)
    _check(load_library().fce_timing_read(arr, cap, ctypes.byref(n)), "fce_timing_read")
    out = {}
    for i in range(min(n.value, cap)):
        out[arr[i].name.decode()] = {"launches": int(arr[i].launches),
                                     "total_ms": float(arr[i].total_ms),
                                     "flops": float(arr[i].flops)}
    return out
