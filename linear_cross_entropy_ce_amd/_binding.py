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
            "fce_fused_fwd_bwd_noalloc", "fce_scale_grads", "fce_get_label_errors",
            "fce_get_filter_stats",
            "fce_status_string",
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
    lib.fce_fused_fwd_bwd_noalloc.restype = i32
    lib.fce_fused_fwd_bwd_noalloc.argtypes = common_ex + [vp, vp, vp, vp]
    lib.fce_scale_grads.restype = i32
    lib.fce_scale_grads.argtypes = [vp, i64, vp, i64, vp, vp]
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


# ---------------------------------------------------------------- checks
# Every wrapper checks its tensors before the library sees a pointer: a CPU
# tensor, one on another device, a non-contiguous view or a mis-sized buffer
# would hand the kernels an address they must not touch.  Errors are
# TypeError (wrong type or dtype) or ValueError (device, layout, shape).
def _tensors(where, **tensors):
    """Each given tensor is a contiguous tensor on the current GPU."""
    import torch

    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{where}: {name} must be a torch.Tensor, not {type(t).__name__}")
        if not t.is_cuda:
            raise ValueError(f"{where}: {name} is on {t.device}; every tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{where}: {name} is on {t.device}, other tensors on {dev}")
    if dev is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"{where}: tensors are on {dev} but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _dtype_is(where, name, t, *dtypes):
    if t is not None and t.dtype not in dtypes:
        raise TypeError(f"{where}: {name} has dtype {t.dtype}; expected "
                        + " or ".join(str(d) for d in dtypes))


def _at_least(where, name, t, n):
    if t is not None and t.numel() < n:
        raise ValueError(f"{where}: {name} holds {t.numel()} elements, needs {n}")


def _shape_is(where, name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _problem(where, X, W, labels):
    """(N, H, V) of X [N, H], W [V, H], labels [N]; X and labels may be None
    for N = 0."""
    import torch

    if W is None:
        raise ValueError(f"{where}: W is required")
    if W.dim() != 2:
        raise ValueError(f"{where}: W must be [V, H], got shape {tuple(W.shape)}")
    _dtype_is(where, "W", W, torch.bfloat16, torch.float32)
    V, H = W.shape
    if X is None:
        if labels is not None and labels.numel() != 0:
            raise ValueError(f"{where}: labels given without X")
        return 0, H, V
    if X.dim() != 2 or X.shape[1] != H:
        raise ValueError(f"{where}: X must be [N, {H}] to match W [{V}, {H}], "
                         f"got shape {tuple(X.shape)}")
    if X.dtype != W.dtype:
        raise TypeError(f"{where}: X ({X.dtype}) and W ({W.dtype}) must share a dtype")
    N = X.shape[0]
    if labels is None:
        raise ValueError(f"{where}: labels are required")
    _dtype_is(where, "labels", labels, torch.int32)
    if labels.numel() != N:
        raise ValueError(f"{where}: labels hold {labels.numel()} elements, X has {N} rows")
    return N, H, V


def _check_call(where, X, W, labels, workspace, reduction, loss=None, lse=None, grad=None,
                dX=None, dW=None, need_loss=False, need_lse=False, need_grads=False):
    import torch

    _tensors(where, X=X, W=W, labels=labels, workspace=workspace, loss=loss, lse=lse,
             grad_loss=grad, dX=dX, dW=dW)
    if workspace is None:
        raise ValueError(f"{where}: a workspace tensor is required")
    N, H, V = _problem(where, X, W, labels)
    none = REDUCTIONS.get(reduction, reduction) == FCE_NONE
    f32 = torch.float32
    for name, t in (("loss", loss), ("lse", lse), ("grad_loss", grad), ("dX", dX), ("dW", dW)):
        _dtype_is(where, name, t, f32)
    if need_loss and (N > 0 or not none):
        if loss is None:
            raise ValueError(f"{where}: loss is required")
        _at_least(where, "loss", loss, N if none else 1)
    if need_lse and N > 0:
        if lse is None:
            raise ValueError(f"{where}: lse is required")
        _at_least(where, "lse", lse, N)
    _at_least(where, "grad_loss", grad, N if none else 1)
    if need_grads:
        if dW is None or (N > 0 and dX is None):
            raise ValueError(f"{where}: dX and dW are required")
        _shape_is(where, "dW", dW, (V, H))
        if N > 0:
            _shape_is(where, "dX", dX, (N, H))
    return N, H, V


def _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule):
    N, H, V = _problem("fce", X, W, labels)
    return [_ptr(X), _ptr(W), _ptr(labels), N, H, V, _dtype_code(W), int(ignore_index),
            float(label_smoothing), REDUCTIONS.get(reduction, reduction), int(chunk),
            SCHEDULES.get(schedule, schedule)]


def fce_forward(X, W, labels, loss, lse, workspace, ignore_index=-100, label_smoothing=0.0,
                reduction="mean", chunk=1024, schedule="auto", stream=None):
    _check_call("fce_forward", X, W, labels, workspace, reduction, loss=loss, lse=lse,
                need_loss=True, need_lse=True)
    args = _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule)
    st = load_library().fce_forward(*args, _ptr(loss), _ptr(lse), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fce_forward")


def fce_backward(X, W, labels, lse, grad_loss, dX, dW, workspace, ignore_index=-100,
                 label_smoothing=0.0, reduction="mean", chunk=1024, schedule="auto", stream=None):
    _check_call("fce_backward", X, W, labels, workspace, reduction, lse=lse, grad=grad_loss,
                dX=dX, dW=dW, need_lse=True, need_grads=True)
    args = _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule)
    st = load_library().fce_backward(*args, _ptr(lse), _ptr(grad_loss), _ptr(dX), _ptr(dW),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check(st, "fce_backward")


def fce_fused_fwd_bwd(X, W, labels, loss, dX, dW, workspace, ignore_index=-100,
                      label_smoothing=0.0, reduction="mean", chunk=1024, schedule="auto",
                      stream=None):
    _check_call("fce_fused_fwd_bwd", X, W, labels, workspace, reduction, loss=loss, dX=dX, dW=dW,
                need_loss=True, need_grads=True)
    args = _common(X, W, labels, ignore_index, label_smoothing, reduction, chunk, schedule)
    st = load_library().fce_fused_fwd_bwd(*args, _ptr(loss), _ptr(dX), _ptr(dW), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream))
    _check(st, "fce_fused_fwd_bwd")


def fce_workspace_size_ex(N, H, V, dtype, **options) -> int:
    o = make_options(**options)
    return int(load_library().fce_workspace_size_ex(N, H, V, dtype, ctypes.byref(o)))


def _common_ex(X, W, labels):
    N, H, V = _problem("fce", X, W, labels)
    return [_ptr(X), _ptr(W), _ptr(labels), N, H, V, _dtype_code(W)]


def _ws(workspace):
    return [_ptr(workspace), workspace.numel() * workspace.element_size()]


def fce_forward_ex(X, W, labels, loss, lse, workspace, stream=None, **options):
    _check_call("fce_forward_ex", X, W, labels, workspace, options.get("reduction", "mean"),
                loss=loss, lse=lse, need_loss=True, need_lse=True)
    o = make_options(**options)
    st = load_library().fce_forward_ex(*_common_ex(X, W, labels), ctypes.byref(o), _ptr(loss),
                                       _ptr(lse), *_ws(workspace), _stream(stream))
    _check(st, "fce_forward_ex")


def fce_backward_ex(X, W, labels, lse, grad_loss, dX, dW, workspace, stream=None, **options):
    _check_call("fce_backward_ex", X, W, labels, workspace, options.get("reduction", "mean"),
                lse=lse, grad=grad_loss, dX=dX, dW=dW, need_lse=True, need_grads=True)
    o = make_options(**options)
    st = load_library().fce_backward_ex(*_common_ex(X, W, labels), ctypes.byref(o), _ptr(lse),
                                        _ptr(grad_loss), _ptr(dX), _ptr(dW), *_ws(workspace),
                                        _stream(stream))
    _check(st, "fce_backward_ex")


def fce_fused_fwd_bwd_ex(X, W, labels, loss, dX, dW, workspace, stream=None, **options):
    _check_call("fce_fused_fwd_bwd_ex", X, W, labels, workspace, options.get("reduction", "mean"),
                loss=loss, dX=dX, dW=dW, need_loss=True, need_grads=True)
    o = make_options(**options)
    st = load_library().fce_fused_fwd_bwd_ex(*_common_ex(X, W, labels), ctypes.byref(o),
                                             _ptr(loss), _ptr(dX), _ptr(dW), *_ws(workspace),
                                             _stream(stream))
    _check(st, "fce_fused_fwd_bwd_ex")


# bytes of the library's static scratch (FCE_STATIC_SCRATCH_BYTES in fce.h)
STATIC_SCRATCH_BYTES = 64 << 20


def fce_fused_fwd_bwd_noalloc(X, W, labels, loss, dX, dW, stream=None, **options):
    """fce_fused_fwd_bwd_ex on the library's static scratch: no workspace
    argument, nothing allocated."""
    _tensors("fce_fused_fwd_bwd_noalloc", X=X, W=W, labels=labels, loss=loss, dX=dX, dW=dW)
    import torch

    N, H, V = _problem("fce_fused_fwd_bwd_noalloc", X, W, labels)
    for name, t in (("loss", loss), ("dX", dX), ("dW", dW)):
        _dtype_is("fce_fused_fwd_bwd_noalloc", name, t, torch.float32)
    none = REDUCTIONS.get(options.get("reduction", "mean"), -1) == FCE_NONE
    if loss is None and (N > 0 or not none):
        raise ValueError("fce_fused_fwd_bwd_noalloc: loss is required")
    _at_least("fce_fused_fwd_bwd_noalloc", "loss", loss, N if none else 1)
    if dW is None or (N > 0 and dX is None):
        raise ValueError("fce_fused_fwd_bwd_noalloc: dX and dW are required")
    _shape_is("fce_fused_fwd_bwd_noalloc", "dW", dW, (V, H))
    if N > 0:
        _shape_is("fce_fused_fwd_bwd_noalloc", "dX", dX, (N, H))
    o = make_options(**options)
    st = load_library().fce_fused_fwd_bwd_noalloc(*_common_ex(X, W, labels), ctypes.byref(o),
                                                  _ptr(loss), _ptr(dX), _ptr(dW),
                                                  _stream(stream))
    _check(st, "fce_fused_fwd_bwd_noalloc")


def fce_ce_logits_workspace_size(N) -> int:
    return int(load_library().fce_ce_logits_workspace_size(N))


def fce_ce_logits(Z, labels, loss, lse, workspace, dZ=None, grad_loss=None, V=None, stream=None,
                  **options):
    """Loss (and dZ, which may be Z) on given logits Z [N, ldz]; V defaults
    to Z's row length."""
    import torch

    where = "fce_ce_logits"
    _tensors(where, Z=Z, labels=labels, loss=loss, lse=lse, workspace=workspace, dZ=dZ,
             grad_loss=grad_loss)
    if Z is None or Z.dim() != 2:
        raise ValueError(f"{where}: Z must be a 2-D [N, ldz] tensor")
    if workspace is None:
        raise ValueError(f"{where}: a workspace tensor is required")
    _dtype_is(where, "Z", Z, torch.bfloat16, torch.float32)
    N, ldz = Z.shape
    V = ldz if V is None else int(V)
    if not 1 <= V <= ldz:
        raise ValueError(f"{where}: V = {V} must lie in [1, {ldz}] (the row length of Z)")
    if labels is None or labels.numel() != N:
        raise ValueError(f"{where}: labels must hold {N} elements (rows of Z)")
    _dtype_is(where, "labels", labels, torch.int32)
    none = REDUCTIONS.get(options.get("reduction", "mean"), -1) == FCE_NONE
    for name, t in (("loss", loss), ("lse", lse), ("grad_loss", grad_loss)):
        _dtype_is(where, name, t, torch.float32)
    if loss is None and (N > 0 or not none):
        raise ValueError(f"{where}: loss is required")
    _at_least(where, "loss", loss, N if none else 1)
    if lse is None and N > 0:
        raise ValueError(f"{where}: lse is required")
    _at_least(where, "lse", lse, N)
    _at_least(where, "grad_loss", grad_loss, N if none else 1)
    if dZ is not None:
        _dtype_is(where, "dZ", dZ, Z.dtype)
        if dZ.dim() != 2 or dZ.shape[0] != N or dZ.shape[1] < V:
            raise ValueError(f"{where}: dZ must be [{N}, >= {V}], got {tuple(dZ.shape)}")
    o = make_options(**options)
    lddz = dZ.shape[1] if dZ is not None else 0
    st = load_library().fce_ce_logits(_ptr(Z), ldz, _ptr(labels), N, V, _dtype_code(Z),
                                      ctypes.byref(o), _ptr(loss), _ptr(lse), _ptr(dZ), lddz,
                                      _ptr(grad_loss), *_ws(workspace), _stream(stream))
    _check(st, "fce_ce_logits")


def fce_scale_grads(dX, dW, grad_loss, stream=None):
    """dX *= g and dW *= g in place, g = grad_loss[0] (a device scalar); dX
    may be None."""
    import torch

    where = "fce_scale_grads"
    _tensors(where, dX=dX, dW=dW, grad_loss=grad_loss)
    for name, t in (("dX", dX), ("dW", dW), ("grad_loss", grad_loss)):
        _dtype_is(where, name, t, torch.float32)
    if dW is None or grad_loss is None:
        raise ValueError(f"{where}: dW and grad_loss are required")
    _at_least(where, "grad_loss", grad_loss, 1)
    n_dx = dX.numel() if dX is not None else 0
    st = load_library().fce_scale_grads(_ptr(dX), n_dx, _ptr(dW), dW.numel(), _ptr(grad_loss),
                                        _stream(stream))
    _check(st, where)


def fce_get_label_errors(workspace, stream=None) -> int:
    _tensors("fce_get_label_errors", workspace=workspace)
    n = ctypes.c_int32(0)
    _check(load_library().fce_get_label_errors(_ptr(workspace), ctypes.byref(n), _stream(stream)),
           "fce_get_label_errors")
    return int(n.value)


def fce_get_filter_stats(workspace, stream=None) -> tuple:
    """(kept, all) dZ tiles of the last filtered backward on this workspace."""
    _tensors("fce_get_filter_stats", workspace=workspace)
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
