"""GPU parity of the loss on given logits (fce_ce_logits) against the fp64
oracle's softmax_ce_on_logits: loss, LSE and dZ element by element, dZ
written in place, into another buffer, or not at all."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linear_cross_entropy_ce_amd as fce  # noqa: E402
import oracle.fce_oracle as orc  # noqa: E402
import parity_log  # noqa: E402
import workloads as wk  # noqa: E402

pytestmark = pytest.mark.gpu

# dZ is stored in the logits' dtype: one bf16 rounding of each element
TOL = {"fp32": (1e-5, 1e-5), "bf16": (2e-3, 1e-2)}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fce.load_library()
    torch.cuda.set_device(0)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def to_np(t):
    return t.float().cpu().numpy()


def run(inp, mode="separate", pad=0, grad=None, **opts):
    """mode: "separate" (dZ in another buffer), "inplace" or "loss" (no dZ)."""
    wl = inp.workload
    Z, y = wk.logits_to_torch(inp, "cuda")
    N, V = Z.shape
    # rows start on 16-byte boundaries: pitch = V rounded up to the vector
    # width, plus `pad` columns
    align = 8 if Z.dtype == torch.bfloat16 else 4
    width = -(-V // align) * align + pad
    if width != V:
        Zp = torch.full((N, width), float("nan"), dtype=Z.dtype, device="cuda")
        Zp[:, :V] = Z
        Z = Zp
    none = opts.get("reduction", "mean") == "none"
    loss = torch.full((N if none else 1,), float("nan"), device="cuda")
    lse = torch.full((max(N, 1),), float("nan"), device="cuda")
    ws = torch.empty(fce.fce_ce_logits_workspace_size(N), dtype=torch.uint8, device="cuda")
    g = None if grad is None else torch.tensor(np.atleast_1d(grad), dtype=torch.float32,
                                               device="cuda")
    dZ = None
    if mode == "separate":
        dZ = torch.full_like(Z, float("nan"))
    elif mode == "inplace":
        dZ = Z
    fce.fce_ce_logits(Z, y, loss, lse, ws, dZ=dZ, grad_loss=g, V=V, **opts)
    torch.cuda.synchronize()
    out = dict(loss=loss.cpu().numpy(), lse=lse[:N].cpu().numpy())
    if dZ is not None:
        out["dZ"] = to_np(dZ[:, :V])
        out["pad"] = to_np(dZ[:, V:])
    return out


def check(inp, got, grad=1.0, tol=None, **opts):
    wl = inp.workload
    red = opts.get("reduction", "mean")
    eps = opts.get("label_smoothing", 0.0)
    loss, lse, dZ = orc.softmax_ce_on_logits(inp.Z, inp.labels, -100, eps, red,
                                             np.asarray(grad, dtype=np.float64),
                                             opts.get("z_loss", 0.0))
    tl, tg = TOL[wl.dtype] if tol is None else tol
    valid = inp.labels != -100
    # relative error with a floor of one nat: with V = 1 every loss is zero
    if red == "none":
        err = np.abs(got["loss"] - loss).max() / max(np.abs(loss[valid]).mean(), 1.0)
    else:
        err = abs(got["loss"][0] - loss) / max(abs(loss), 1.0)
    el = rel_l2(got["lse"][valid], lse[valid])
    label = f"ce_logits {wl.name} {wl.N}x{wl.V} {wl.dtype} {red}"
    print(f"[{label}] loss {err:.2e} lse {el:.2e}", end="", flush=True)
    errs = dict(loss=err, lse=el)
    if "dZ" in got:
        # a row's dZ has norm of order s_i, the row's gradient scale (g / D,
        # or g_i for reduction none); the relative error's denominator is
        # floored at 1% of ||s||, for V = 1 where dZ is zero up to rounding
        g = np.broadcast_to(np.asarray(grad, dtype=np.float64), (wl.N,)) if red == "none" \
            else np.full(wl.N, float(grad) / (max(int(valid.sum()), 1) if red == "mean" else 1))
        floor = 1e-2 * np.linalg.norm(np.where(valid, g, 0.0))
        ed = np.linalg.norm(got["dZ"].astype(np.float64) - dZ) / max(np.linalg.norm(dZ), floor)
        print(f" dZ {ed:.2e}", flush=True)
        errs["dZ"] = ed
    else:
        print(flush=True)
    parity_log.record(label, tl, tg, **errs)
    assert err <= tl and el <= tl
    if "dZ" in got:
        assert errs["dZ"] <= tg
        assert np.all(got["dZ"][~valid] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["separate", "inplace", "loss"])
def test_modes(dtype, mode):
    wl = wk.custom(300, 64, 5003, dtype, 0.05, "zipf", 1.1, 0.05, 0.0, seed=81)
    inp = wk.draw_logits(wl)
    got = run(inp, mode=mode)
    check(inp, got)


@pytest.mark.parametrize("red", ["mean", "sum", "none"])
def test_reductions_zloss_smoothing(red):
    wl = wk.custom(257, 256, 4099, "bf16", 0.04, "uniform", 1.1, 0.1, 0.0, seed=83)
    inp = wk.draw_logits(wl)
    g = np.random.default_rng(4).uniform(-2, 2, wl.N).astype(np.float32) if red == "none" else 0.6
    opts = dict(reduction=red, z_loss=1e-3, label_smoothing=0.1)
    got = run(inp, grad=g, **opts)
    check(inp, got, grad=g, **opts)


@pytest.mark.parametrize("V", [1, 7, 8, 9, 1000, 8193, 70001, 140001])
def test_ragged_rows_and_padding(V):
    wl = wk.custom(33, 16, V, "bf16", 0.5, "uniform", 1.1, 0.1, 0.0, seed=85 + V)
    inp = wk.draw_logits(wl)
    got = run(inp, pad=8, label_smoothing=0.05)
    check(inp, got, label_smoothing=0.05)
    # columns past V inside the last 16-byte vector are zeroed; the rest of
    # the padding is untouched (it was NaN)
    tail = (-V) % 8
    assert np.all(got["pad"][:, :tail] == 0.0)
    assert np.all(np.isnan(got["pad"][:, tail:]))


@pytest.mark.parametrize("V", [5003, 40000])
def test_fp32_rows(V):
    wl = wk.custom(70, 64, V, "fp32", 0.05, "uniform", 1.1, 0.1, 0.0, seed=97)
    inp = wk.draw_logits(wl)
    got = run(inp, label_smoothing=0.1, z_loss=1e-3)
    check(inp, got, label_smoothing=0.1, z_loss=1e-3)


def test_invalid_and_ignored_rows():
    wl = wk.custom(64, 16, 500, "bf16", 0.5, "uniform", 1.1, 0.25, 0.0, seed=87)
    inp = wk.draw_logits(wl)
    inp.labels[5] = 500  # outside [0, V), not ignore_index
    got = run(inp, reduction="none")
    assert np.isnan(got["loss"][5])
    assert np.all(got["loss"][inp.labels == -100] == 0.0)
    got = run(inp)
    assert np.isnan(got["loss"][0])


def test_large_logits_stay_finite():
    wl = wk.custom(40, 4096, 3000, "fp32", 2.0, "uniform", seed=89)  # logit sd ~ 128
    inp = wk.draw_logits(wl)
    got = run(inp)
    assert np.isfinite(got["loss"]).all() and np.isfinite(got["dZ"]).all()
    # |LSE| is in the hundreds: the kernel keeps the row max m and log2 of
    # the sum apart and forms each exponent as (z - m) log2e - log2 l, exact
    # near the max, so fp32's 1e-5 holds here as for small logits
    print(f"|LSE| up to {np.abs(got['lse']).max():.0f}")
    check(inp, got)


@pytest.mark.parametrize("dtype,V", [("bf16", 70001), ("fp32", 40000)])
@pytest.mark.parametrize("mode", ["separate", "loss"])
def test_rows_whose_maximum_climbs(dtype, V, mode):
    # Each thread's reference point moves when a later vector's maximum
    # passes it by more than 16 nats: rows that climb 200 nats from left to
    # right move it at every iteration, falling rows never after the first,
    # and a late spike of 60 nats over the row moves it once, far.
    wl = wk.custom(48, 64, V, dtype, 0.02, "uniform", 1.1, 0.1, 0.0, seed=91)
    inp = wk.draw_logits(wl)
    ramp = np.linspace(0.0, 200.0, V, dtype=np.float32)
    Z = inp.Z
    Z[0::3] += ramp
    Z[1::3] += ramp[::-1]
    Z[2::3, V - 37] += 60.0
    if dtype == "bf16":
        inp.Z_bits = wk.round_to_bf16_bits(Z)
        inp.Z = wk.bf16_bits_to_f32(inp.Z_bits)
    got = run(inp, mode=mode, label_smoothing=0.05)
    check(inp, got, label_smoothing=0.05)


def test_full_size_llama2_shape():
    # 4096 x 32000 logits (the 4096x2048x32000 workload's logit shape), every element
    inp = wk.draw_logits(wk.WORKLOADS[2])
    got = run(inp, mode="inplace")
    check(inp, got)


def test_full_size_llama3_shape_sampled_rows():
    # 8192 x 128256: LSE and dZ of sampled rows against the oracle; the loss
    # against the per-row terms of those rows is covered by the smaller cases
    inp = wk.draw_logits(wk.WORKLOADS[3])
    got = run(inp, mode="inplace", reduction="none")
    rows = np.random.default_rng(3).choice(inp.workload.N, 48, replace=False)
    loss, lse, dZ = orc.softmax_ce_on_logits(inp.Z[rows], inp.labels[rows], -100, 0.0, "none")
    v = inp.labels[rows] != -100
    assert np.abs(got["loss"][rows] - loss).max() <= 2e-3 * np.abs(loss[v]).mean()
    assert rel_l2(got["lse"][rows][v], lse[v]) <= 2e-3
    assert rel_l2(got["dZ"][rows], dZ) <= 1e-2
