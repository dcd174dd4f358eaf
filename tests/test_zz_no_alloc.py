"""GPU test of fce_fused_fwd_bwd_noalloc, the entry point that allocates
nothing: it runs fce_fused_fwd_bwd_ex's kernels on the library's static
scratch.  Two calls in a row (the second on a smaller input, so the scratch
holds the first call's bytes when it starts), each compared bitwise with
fce_fused_fwd_bwd_ex on a workspace of its own, and against the fp64 oracle
to the bf16 tolerance."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linear_cross_entropy_ce_amd as fce  # noqa: E402
import oracle.fce_oracle as orc  # noqa: E402
import workloads as wk  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fce.load_library()
    torch.cuda.set_device(0)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _both(inp, **opts):
    wl = inp.workload
    X, W, y = wk.to_torch(inp, "cuda")
    N, H, V = wl.N, wl.H, wl.V
    code = fce.FCE_BF16 if X.dtype == torch.bfloat16 else fce.FCE_F32
    need = fce.fce_workspace_size_ex(N, H, V, code, **opts)
    assert 0 < need <= fce.STATIC_SCRATCH_BYTES, need
    outs = []
    for noalloc in (False, True):
        loss = torch.full((1,), float("nan"), device="cuda")
        dX = torch.full((N, H), float("nan"), device="cuda")
        dW = torch.full((V, H), float("nan"), device="cuda")
        if noalloc:
            fce.fce_fused_fwd_bwd_noalloc(X, W, y, loss, dX, dW, **opts)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            fce.fce_fused_fwd_bwd_ex(X, W, y, loss, dX, dW, ws, **opts)
        torch.cuda.synchronize()
        outs.append((loss.item(), dX.cpu().numpy(), dW.cpu().numpy()))
    return outs


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    cases = [
        (wk.custom(900, 256, 4000, "bf16", 0.03, "zipf", 1.1, 0.05, 0.1, seed=201),
         dict(chunk=300, label_smoothing=0.1, z_loss=1e-4)),
        (wk.custom(300, 64, 1500, "bf16", 0.05, "uniform", ignore_frac=0.1, seed=203),
         dict(chunk=128)),  # smaller: the scratch still holds the first call's bytes
    ]
    for wl, opts in cases:
        print(f"[noalloc] {wl.N}x{wl.H}x{wl.V} {wl.dtype} {opts}", flush=True)
        inp = wk.draw(wl)
        (l0, x0, w0), (l1, x1, w1) = _both(inp, **opts)
        assert l0 == l1 and np.array_equal(x0, x1) and np.array_equal(w0, w1)
        ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100,
                                       opts.get("label_smoothing", 0.0), "mean", 1.0,
                                       z_loss=opts.get("z_loss", 0.0))
        assert abs(l1 - ref.loss) <= 2e-3 * abs(ref.loss)
        assert rel_l2(x1, ref.dX) <= 2e-2 and rel_l2(w1, ref.dW) <= 2e-2


def test_noalloc_rejects_a_problem_over_the_scratch_size():
    wl = wk.custom(512, 256, 70000, "bf16", seed=205)
    X = torch.zeros((wl.N, wl.H), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((wl.V, wl.H), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(wl.N, dtype=torch.int32, device="cuda")
    loss = torch.empty(1, device="cuda")
    dX = torch.empty((wl.N, wl.H), device="cuda")
    dW = torch.empty((wl.V, wl.H), device="cuda")
    assert fce.fce_workspace_size_ex(wl.N, wl.H, wl.V, fce.FCE_BF16,
                                     chunk=4096) > fce.STATIC_SCRATCH_BYTES
    with pytest.raises(fce.FceError, match="workspace"):
        fce.fce_fused_fwd_bwd_noalloc(X, W, y, loss, dX, dW, chunk=4096)
