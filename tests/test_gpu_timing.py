"""GPU: the library's per-kernel timing (fce_timing_enable / fce_timing_read).

Within one call consecutive kernels share the event between them, and each
call starts a chain of its own.  Checked here: every kernel family of the
fused step is reported with the launch count the plan implies, its FLOPs,
positive durations, and a sum of kernel times that fits inside the calls'
own wall-clock interval; work the caller enqueues between two calls is not
charged to any kernel.
"""
import pytest

torch = pytest.importorskip("torch")

import linear_cross_entropy_ce_amd as fce  # noqa: E402
import workloads as wk  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fce.load_library()
    torch.cuda.set_device(0)


def test_fused_step_timing_counts_and_sums():
    wl = wk.custom(1500, 512, 9000, "bf16", 0.03, "uniform", ignore_frac=0.02, seed=101)
    inp = wk.draw(wl)
    X, W, y = wk.to_torch(inp, "cuda")
    N, H, V = wl.N, wl.H, wl.V
    chunk = 512
    plan = fce.fce_plan(N, H, V, 1, chunk)
    blocks = plan["n_token_blocks"] * plan["n_vocab_blocks"]
    ws = fce.workspace_for(N, H, V, X.dtype, chunk)
    loss = torch.empty(1, device="cuda")
    dX = torch.empty((N, H), device="cuda")
    dW = torch.empty((V, H), device="cuda")

    def step():
        fce.fce_fused_fwd_bwd(X, W, y, loss, dX, dW, ws, -100, 0.0, "mean", chunk)

    step()
    torch.cuda.synchronize()
    calls = 3
    junk = torch.empty(64 << 20, device="cuda")
    fce.fce_timing_enable(True)
    try:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            step()
            junk.mul_(1.0001)  # caller's work between calls: not any kernel's
        b.record()
        torch.cuda.synchronize()
        kern = fce.fce_timing_read()
    finally:
        fce.fce_timing_enable(False)
    wall = a.elapsed_time(b)
    for name in ("label_scan", "fwd_lse", "lse_merge", "loss_final"):
        assert kern[name]["launches"] == calls, (name, kern[name])
    # bf16, unfiltered: dW and dX of a logit block share one launch
    assert "bwd_dw" not in kern and "bwd_dx" not in kern
    for name in ("bwd_dz", "bwd_grad"):
        assert kern[name]["launches"] == calls * blocks, (name, kern[name], blocks)
    for name, r in kern.items():
        assert r["total_ms"] > 0.0, (name, r)
    assert kern["fwd_lse"]["flops"] == pytest.approx(calls * 2.0 * N * V * H, rel=1e-9)
    assert kern["bwd_dz"]["flops"] == pytest.approx(calls * 2.0 * N * V * H, rel=1e-9)
    assert kern["bwd_grad"]["flops"] == pytest.approx(calls * 4.0 * N * V * H, rel=1e-9)
    total = sum(r["total_ms"] for r in kern.values())
    # the junk work ran between calls: time that no kernel may have absorbed
    j0 = torch.cuda.Event(enable_timing=True)
    j1 = torch.cuda.Event(enable_timing=True)
    j0.record()
    for _ in range(calls):
        junk.mul_(1.0001)
    j1.record()
    torch.cuda.synchronize()
    junk_ms = j0.elapsed_time(j1)
    print(f"[timing] wall {wall:.3f} ms, kernels {total:.3f} ms, caller's work {junk_ms:.3f} ms",
          flush=True)
    assert total <= wall - 0.5 * junk_ms, (total, wall, junk_ms)
    # the first kernel of each call starts its own interval: had it reused
    # the previous call's last event, it would hold the caller's work
    assert kern["label_scan"]["total_ms"] < 0.5 * junk_ms, (kern["label_scan"], junk_ms)
    # a read resets the counters
    assert fce.fce_timing_read() == {}
