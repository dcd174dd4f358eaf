"""Host-only checks of the Python binding's argument validation (no GPU).

Every wrapper checks its tensors before the library sees a pointer: CPU
tensors, mismatched shapes and wrong dtypes are a Python error, not a device
address handed to a kernel."""
import pytest

torch = pytest.importorskip("torch")

import linear_cross_entropy_ce_amd as fce  # noqa: E402
from linear_cross_entropy_ce_amd import _binding as B  # noqa: E402


def _cpu_problem(N=8, H=16, V=32, dtype=torch.bfloat16):
    X = torch.zeros(N, H, dtype=dtype)
    W = torch.zeros(V, H, dtype=dtype)
    y = torch.zeros(N, dtype=torch.int32)
    return X, W, y


def test_cpu_tensors_are_rejected_before_any_library_call():
    X, W, y = _cpu_problem()
    loss = torch.zeros(1)
    lse = torch.zeros(8)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        fce.fce_forward(X, W, y, loss, lse, ws)
    with pytest.raises(ValueError, match="GPU"):
        fce.fce_fused_fwd_bwd_ex(X, W, y, loss, torch.zeros(8, 16), torch.zeros(32, 16), ws)
    with pytest.raises(ValueError, match="GPU"):
        fce.fce_ce_logits(torch.zeros(8, 32), y, loss, lse, ws)
    with pytest.raises(ValueError, match="GPU"):
        fce.fce_scale_grads(torch.zeros(8, 16), torch.zeros(32, 16), torch.ones(1))
    with pytest.raises(ValueError, match="GPU"):
        fce.fce_get_label_errors(ws)


def test_autograd_wrapper_rejects_cpu_inputs():
    X, W, y = _cpu_problem(dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        fce.linear_cross_entropy(X, W, y.long())


def test_problem_shapes_and_dtypes():
    X, W, y = _cpu_problem()
    assert B._problem("t", X, W, y) == (8, 16, 32)
    assert B._problem("t", None, W, None) == (0, 16, 32)
    with pytest.raises(ValueError, match="X must be"):
        B._problem("t", torch.zeros(8, 24, dtype=torch.bfloat16), W, y)  # H mismatch
    with pytest.raises(ValueError, match="W must be"):
        B._problem("t", X, torch.zeros(32, dtype=torch.bfloat16), y)
    with pytest.raises(ValueError, match="labels hold"):
        B._problem("t", X, W, torch.zeros(7, dtype=torch.int32))
    with pytest.raises(TypeError, match="labels"):
        B._problem("t", X, W, torch.zeros(8, dtype=torch.int64))
    with pytest.raises(TypeError, match="share a dtype"):
        B._problem("t", X.float(), W, y)
    with pytest.raises(TypeError, match="W"):
        B._problem("t", X.half(), W.half(), y)


def test_output_sizes():
    with pytest.raises(ValueError, match="shape"):
        B._shape_is("t", "dW", torch.zeros(31, 16), (32, 16))
    with pytest.raises(ValueError, match="needs 8"):
        B._at_least("t", "lse", torch.zeros(7), 8)
    with pytest.raises(TypeError, match="float32"):
        B._dtype_is("t", "dX", torch.zeros(2, dtype=torch.bfloat16), torch.float32)


def test_non_contiguous_and_non_tensor_arguments():
    with pytest.raises(TypeError, match="torch.Tensor"):
        B._tensors("t", X=[1, 2, 3])
    # contiguity is checked after the device: a CPU view fails on the device first
    with pytest.raises(ValueError):
        B._tensors("t", X=torch.zeros(4, 4).t())


def test_scale_entry_point_rejects_bad_arguments_without_launching():
    lib = B.load_library()
    FAKE = 0x10000
    assert lib.fce_scale_grads(FAKE, -1, FAKE, 4, FAKE, None) == B.FCE_ERR_SHAPE
    assert lib.fce_scale_grads(FAKE, 4, FAKE, 4, None, None) == B.FCE_ERR_NULL
    assert lib.fce_scale_grads(None, 4, FAKE, 4, FAKE, None) == B.FCE_ERR_NULL
    assert lib.fce_scale_grads(FAKE + 4, 4, FAKE, 4, FAKE, None) == B.FCE_ERR_ALIGN
    assert lib.fce_scale_grads(None, 0, None, 0, FAKE, None) == B.FCE_OK  # nothing to do
