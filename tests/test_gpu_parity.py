"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Small cases are compared element by element with the full oracle.  At full
size the 4096 x 2048 x 32000 workload is compared whole: the oracle runs at
test time.  The three larger workloads are compared on the loss and every
row's LSE (stored by tests/golden/make_oracle_goldens.py), and on dX and dW
rows the oracle computes at test time: in every 256-row tile of dX and of dW,
the tile's first and last row and one drawn at random.  Every block boundary
of every plan falls on a tile boundary, so both sides of each are compared.
Tolerances (relative error of the loss, relative L2 error of dX and dW): 1e-5
for fp32 inputs; 2e-3 (loss) and 2e-2 (gradients) for bf16 inputs, whose only
rounding in the library beyond fp32 is the bf16 store of the softmax-minus-
target block.  Every measured error is printed at the end of the run.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linear_cross_entropy_ce_amd as fce  # noqa: E402
import oracle.fce_oracle as orc  # noqa: E402
import parity_log  # noqa: E402
import workloads as wk  # noqa: E402

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = {"fp32": (1e-5, 1e-5), "bf16": (2e-3, 2e-2)}


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


def run(inp, chunk=1024, schedule="auto", eps=None, reduction="mean", split=False, grad=None):
    """Run the library on a drawn input; returns loss, lse, dX, dW as numpy."""
    wl = inp.workload
    eps = wl.label_smoothing if eps is None else eps
    X, W, y = wk.to_torch(inp, "cuda")
    N, H, V = wl.N, wl.H, wl.V
    ws = fce.workspace_for(N, H, V, X.dtype, chunk, schedule)
    loss = torch.full((1,), float("nan"), device="cuda")
    lse = torch.full((max(N, 1),), float("nan"), device="cuda")
    dX = torch.full((max(N, 1), H), float("nan"), device="cuda")
    dW = torch.full((V, H), float("nan"), device="cuda")
    Xp, yp, dXp = (X, y, dX) if N > 0 else (None, None, None)
    if split or grad is not None:
        g = None if grad is None else torch.tensor([grad], dtype=torch.float32, device="cuda")
        fce.fce_forward(Xp, W, yp, loss, lse, ws, -100, eps, reduction, chunk, schedule)
        fce.fce_backward(Xp, W, yp, lse, g, dXp, dW, ws, -100, eps, reduction, chunk, schedule)
    else:
        fce.fce_fused_fwd_bwd(Xp, W, yp, loss, dXp, dW, ws, -100, eps, reduction, chunk, schedule)
        # the fused call keeps the LSE in its workspace: fetch it from the forward entry point
        loss2 = torch.empty(1, device="cuda")
        fce.fce_forward(Xp, W, yp, loss2, lse, ws, -100, eps, reduction, chunk, schedule)
    torch.cuda.synchronize()
    errors = fce.fce_get_label_errors(ws)
    return dict(loss=loss.item(), lse=lse[:N].cpu().numpy(), dX=dX[:N].cpu().numpy(),
                dW=dW.cpu().numpy(), label_errors=errors)


def check_against_oracle(inp, got, eps=None, reduction="mean", grad=1.0, tol=None, name=None):
    wl = inp.workload
    eps = wl.label_smoothing if eps is None else eps
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, eps, reduction, grad)
    tl, tg = tol or TOL[wl.dtype]
    le = abs(got["loss"] - ref.loss) / max(abs(ref.loss), 1e-30)
    ex = rel_l2(got["dX"], ref.dX)
    ew = rel_l2(got["dW"], ref.dW)
    valid = inp.labels != -100
    el = (rel_l2(got["lse"][valid], ref.lse[valid])
          if got["lse"].size and valid.any() else 0.0)
    label = name or f"{wl.name} {wl.N}x{wl.H}x{wl.V} {wl.dtype}"
    print(f"[{label}] loss {got['loss']:.7f} vs {ref.loss:.7f} "
          f"rel {le:.2e}; lse {el:.2e}; dX rel-L2 {ex:.2e}; dW rel-L2 {ew:.2e}", flush=True)
    parity_log.record(label, tl, tg, loss=le, lse=el, dX=ex, dW=ew)
    assert le <= tl, (got["loss"], ref.loss)
    assert ex <= tg and ew <= tg, (ex, ew)
    assert el <= tl
    # ignored rows have exactly zero gradient
    assert np.all(got["dX"][~valid] == 0.0)
    return ref


# ------------------------------------------------------------ small shapes
def test_tiny_fp32_workload():
    inp = wk.draw(wk.WORKLOADS[1])
    check_against_oracle(inp, run(inp))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_shapes_with_smoothing_and_ignore(dtype):
    wl = wk.custom(700, 264 if dtype == "bf16" else 36, 5003, dtype, 0.05, "zipf", 1.1, 0.05, 0.1,
                   seed=31)
    inp = wk.draw(wl)
    check_against_oracle(inp, run(inp, chunk=300))


@pytest.mark.parametrize("schedule", ["token", "vocab", "auto"])
def test_schedules_agree(schedule):
    wl = wk.custom(1000, 128, 3000, "bf16", 0.05, "uniform", ignore_frac=0.1, label_smoothing=0.0,
                   seed=41)
    inp = wk.draw(wl)
    got = run(inp, chunk=300, schedule=schedule)
    check_against_oracle(inp, got)
    base = run(inp, chunk=100000)  # one block
    assert abs(got["loss"] - base["loss"]) <= 1e-6 * abs(base["loss"])
    assert rel_l2(got["dX"], base["dX"]) <= 1e-5 and rel_l2(got["dW"], base["dW"]) <= 1e-5


def test_sum_reduction_and_upstream_gradient():
    wl = wk.custom(300, 64, 1500, "fp32", 0.1, "uniform", ignore_frac=0.1, label_smoothing=0.2,
                   seed=43)
    inp = wk.draw(wl)
    got = run(inp, chunk=128, reduction="sum", grad=2.5)
    check_against_oracle(inp, got, reduction="sum", grad=2.5)


def test_split_calls_equal_fused_bitwise_and_runs_are_deterministic():
    wl = wk.custom(900, 256, 4000, "bf16", 0.03, "zipf", 1.1, 0.03, 0.1, seed=47)
    inp = wk.draw(wl)
    a = run(inp, chunk=200)
    b = run(inp, chunk=200)
    c = run(inp, chunk=200, split=True)
    for k in ("dX", "dW"):
        assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k])
    assert a["loss"] == b["loss"] == c["loss"]


def test_all_labels_ignored():
    wl = wk.custom(300, 64, 700, "bf16", seed=51, ignore_frac=1.0)
    inp = wk.draw(wl)
    got = run(inp, chunk=64)
    assert got["loss"] == 0.0
    assert not got["dX"].any() and not got["dW"].any()


@pytest.mark.parametrize("H,block", [(64, 0), (256, 0), (256, 1)])
def test_one_token_block_all_ignored(H, block):
    # H = 64 takes the per-tile dZ kernel, H = 256 the streamed one; with the
    # middle block ignored, dW is accumulated both before and after it
    wl = wk.custom(700, H, 3000, "bf16", seed=53, ignore_frac=0.0)
    inp = wk.draw(wl)
    inp.labels[256 * block:256 * (block + 1)] = -100  # one 256-token block has no valid label
    got = run(inp, chunk=256, schedule="token")
    check_against_oracle(inp, got)


@pytest.mark.parametrize("H,variant", [(384, "recompute"), (320, "store_logits")])
def test_transposed_dw_over_accumulating_token_blocks(H, variant):
    # token blocks of 8192 take dW as X^T dZ: three blocks (8192, 8192, 300)
    # accumulate into dW, with a partial H tile and a partial vocabulary tile
    wl = wk.custom(2 * 8192 + 300, H, 2000, "bf16", ignore_frac=0.1, seed=61)
    inp = wk.draw(wl)
    if variant == "recompute":
        got = run(inp, chunk=8192, schedule="token")
    else:
        got = run_ex(inp, split=False, chunk=8192, variant="store_logits")
        # the fused store-logits call returns the loss; its LSE stays in the workspace
        got["loss"] = float(got["loss"][0])
        got["lse"] = np.empty(0)
    check_against_oracle(inp, got)


def test_empty_batch():
    wl = wk.custom(0, 64, 700, "bf16", seed=55)
    inp = wk.draw(wl)
    got = run(inp)
    assert got["loss"] == 0.0 and not got["dW"].any()


@pytest.mark.parametrize("N,H,V", [(1, 8, 1), (1, 16, 3), (5, 8, 2), (33, 8, 257), (257, 520, 300)])
def test_degenerate_shapes(N, H, V):
    wl = wk.custom(N, H, V, "bf16", 0.5, seed=57 + N)
    inp = wk.draw(wl)
    ref = check_against_oracle(inp, run(inp, chunk=7))
    if V == 1:
        assert ref.loss == 0.0


def test_invalid_label_is_reported():
    wl = wk.custom(200, 64, 500, "bf16", seed=59)
    inp = wk.draw(wl)
    inp.labels[7] = 500  # == V: out of range and not ignore_index
    got = run(inp)
    assert got["label_errors"] == 1
    assert np.isnan(got["loss"])
    assert np.all(got["dX"][7] == 0.0)


def test_large_logits_stay_finite():
    wl = wk.custom(400, 128, 2000, "bf16", 0.5, seed=61)
    inp = wk.draw(wl)
    # X * 64 is exact in bf16; logits reach the thousands
    inp.X_bits = wk.round_to_bf16_bits(inp.X * 64)
    inp.X = wk.bf16_bits_to_f32(inp.X_bits)
    got = run(inp)
    assert np.isfinite(got["loss"]) and np.isfinite(got["dX"]).all() and np.isfinite(got["dW"]).all()
    check_against_oracle(inp, got)


@pytest.mark.parametrize("n", [0, 1, 5, 1001, 1 << 20])
def test_scale_grads_entry_point(n):
    # dX *= g and dW *= g in place (one IEEE multiply each: bitwise torch's)
    gen = torch.Generator(device="cuda").manual_seed(n)
    dX = torch.randn(n, device="cuda", generator=gen)
    dW = torch.randn(n + 3, device="cuda", generator=gen)
    g = torch.tensor([0.37], device="cuda")
    ex, ew = dX * g, dW * g
    fce.fce_scale_grads(dX if n else None, dW, g)
    torch.cuda.synchronize()
    assert torch.equal(dX, ex) and torch.equal(dW, ew)


# fp32 at large logits.  The fused call keeps the forward's row statistics
# split (row max m and log2 of the sum of exp(z - m)) and forms every
# exponent as (z - m) log2e - log2 l, which is exact near the max whatever
# |LSE| is; the loss term is (m - z_y) + log l.  Three regimes: logit spread
# of about 64 and 256 (|LSE| about 200 and 900, softmax close to one-hot),
# and logits of spread ~0.6 on a common offset of 300 (|LSE| about 308,
# softmax spread over many entries; the offset cancels in the math but not
# in fp32).  The fp32 rounding of the logits themselves costs about 3e-6 of
# relative L2 in these cases (an fp32 GEMM of the same inputs, evaluated in
# fp64 on the CPU), so 1e-5 holds with margin.
def _fp32_large(kind):
    if kind == "offset":
        wl = wk.custom(400, 128, 2000, "fp32", 0.05, ignore_frac=0.05, seed=63,
                       name="fp32-offset300")
        inp = wk.draw(wl)
        inp.X[:, 0] = 1.0
        inp.W[:, 0] = 300.0
    else:
        scale = {"x16": 16.0, "x64": 64.0}[kind]
        wl = wk.custom(400, 64, 2000, "fp32", 0.5, ignore_frac=0.05, seed=65,
                       name=f"fp32-spread-{kind}")
        inp = wk.draw(wl)
        inp.X *= np.float32(scale)  # a power of two: exact
    return inp


def _check_fp32_large(inp, got, kind, tg, name):
    """check_against_oracle, except that with the offset dX column 0 is
    checked on its own: it is 300 times the row sums of dZ, exactly 0 in
    real arithmetic, so in fp32 it holds 300 times their rounding, and its
    relative error is not defined by the method (any fp32 dX = dZ W has it).
    The other columns and dW are held to the bound."""
    if kind != "offset":
        return check_against_oracle(inp, got, tol=(1e-5, tg), name=name)
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, 0.0, "mean")
    valid = inp.labels != -100
    le = abs(got["loss"] - ref.loss) / abs(ref.loss)
    el = rel_l2(got["lse"][valid], ref.lse[valid])
    ex = rel_l2(got["dX"][:, 1:], ref.dX[:, 1:])
    ew = rel_l2(got["dW"], ref.dW)
    col0 = np.linalg.norm(got["dX"][:, 0]) / np.linalg.norm(got["dX"][:, 1:])
    print(f"[{name}] loss {le:.2e} lse {el:.2e} dX (columns 1..) {ex:.2e} dW {ew:.2e}; "
          f"|dX[:, 0]| / |dX[:, 1:]| {col0:.2e}", flush=True)
    parity_log.record(name, 1e-5, tg, loss=le, lse=el, dX_cols_1_on=ex, dW=ew)
    assert le <= 1e-5 and el <= 1e-5 and ex <= tg and ew <= tg
    assert col0 <= 1e-2  # 300 x the rounding of sums that are 0, small beside the rest


@pytest.mark.parametrize("kind", ["x16", "x64", "offset"])
def test_fp32_large_logits_fused(kind):
    inp = _fp32_large(kind)
    got = run(inp, chunk=128)
    lse = got["lse"][inp.labels != -100]
    print(f"[{inp.workload.name}] |LSE| from {np.abs(lse).min():.0f} to {np.abs(lse).max():.0f}")
    _check_fp32_large(inp, got, kind, 1e-5, f"{inp.workload.name} fused")


# The split calls hand the LSE from fce_forward to fce_backward as one fp32
# value per row, rounded to within |LSE| 2^-25: every probability of the row
# is then off by a factor within exp(|LSE| 2^-25), so the gradients carry a
# relative error up to about |LSE| 2^-25 beyond the fused call's (a property
# of the fp32 lse argument, not of the kernels).  Bound: the fp32 tolerance
# or 2 max|LSE| 2^-24, whichever is larger.
@pytest.mark.parametrize("kind", ["x16", "x64", "offset"])
def test_fp32_large_logits_split_calls(kind):
    inp = _fp32_large(kind)
    got = run(inp, chunk=128, split=True)
    tg = max(1e-5, 2.0 * np.nanmax(np.abs(got["lse"])) * 2.0 ** -24)
    _check_fp32_large(inp, got, kind, tg, f"{inp.workload.name} split")


def test_autograd_wrapper():
    wl = wk.custom(3 * 130, 64, 900, "fp32", 0.1, ignore_frac=0.1, label_smoothing=0.1, seed=67)
    inp = wk.draw(wl)
    X, W, y = wk.to_torch(inp, "cuda")
    Xr = X.reshape(3, 130, 64).clone().requires_grad_(True)
    Wr = W.clone().requires_grad_(True)
    loss = fce.linear_cross_entropy(Xr, Wr, y.reshape(3, 130).long(), label_smoothing=0.1, chunk=100)
    (loss * 0.5).backward()
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, 0.1, "mean", 0.5)
    assert abs(loss.item() - ref.loss) <= 1e-5 * ref.loss
    assert rel_l2(Xr.grad.reshape(-1, 64).cpu().numpy(), ref.dX) <= 1e-5
    assert rel_l2(Wr.grad.cpu().numpy(), ref.dW) <= 1e-5


@pytest.mark.parametrize("dtype,variant", [("fp32", "store_logits"), ("bf16", "store_logits"),
                                           ("bf16", "filtered")])
def test_autograd_wrapper_variants(dtype, variant):
    # the gradients of the store-logits variant are computed in the forward
    # and scaled by the upstream gradient (0.5 here) in the backward
    wl = wk.custom(3 * 130, 64, 900, dtype, 0.1, ignore_frac=0.1, label_smoothing=0.1, seed=69)
    inp = wk.draw(wl)
    X, W, y = wk.to_torch(inp, "cuda")
    Xr = X.reshape(3, 130, 64).clone().requires_grad_(True)
    Wr = W.clone().requires_grad_(True)
    loss = fce.linear_cross_entropy(Xr, Wr, y.reshape(3, 130).long(), label_smoothing=0.1,
                                    chunk=100, z_loss=1e-3, variant=variant)
    (loss * 0.5).backward()
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, 0.1, "mean", 0.5, z_loss=1e-3)
    tl, tg = TOL[dtype]
    assert abs(loss.item() - ref.loss) <= tl * ref.loss
    assert rel_l2(Xr.grad.reshape(-1, 64).float().cpu().numpy(), ref.dX) <= tg
    assert rel_l2(Wr.grad.float().cpu().numpy(), ref.dW) <= tg


# ------------------------------------------- z-loss and reduction "none"
def run_ex(inp, grad=None, split=True, **opts):
    """The *_ex entry points; grad: per-token array for "none", scalar else."""
    wl = inp.workload
    X, W, y = wk.to_torch(inp, "cuda")
    N, H, V = wl.N, wl.H, wl.V
    opts.setdefault("label_smoothing", wl.label_smoothing)
    code = fce.FCE_BF16 if X.dtype == torch.bfloat16 else fce.FCE_F32
    ws = torch.empty(fce.fce_workspace_size_ex(N, H, V, code, **opts), dtype=torch.uint8,
                     device="cuda")
    none = opts.get("reduction", "mean") == "none"
    loss = torch.full((N if none else 1,), float("nan"), device="cuda")
    lse = torch.full((max(N, 1),), float("nan"), device="cuda")
    dX = torch.full((max(N, 1), H), float("nan"), device="cuda")
    dW = torch.full((V, H), float("nan"), device="cuda")
    if split:
        g = None if grad is None else torch.tensor(np.atleast_1d(grad), dtype=torch.float32,
                                                   device="cuda")
        fce.fce_forward_ex(X, W, y, loss, lse, ws, **opts)
        fce.fce_backward_ex(X, W, y, lse, g, dX, dW, ws, **opts)
    else:
        fce.fce_fused_fwd_bwd_ex(X, W, y, loss, dX, dW, ws, **opts)
    torch.cuda.synchronize()
    return dict(loss=loss.cpu().numpy(), lse=lse[:N].cpu().numpy(), dX=dX[:N].cpu().numpy(),
                dW=dW.cpu().numpy())


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_zloss_and_reductions(dtype, reduction):
    wl = wk.custom(700, 264 if dtype == "bf16" else 36, 5003, dtype, 0.05, "zipf", 1.1, 0.05, 0.1,
                   seed=71)
    inp = wk.draw(wl)
    al = 1e-3
    g = (np.random.default_rng(5).uniform(-2.0, 2.0, wl.N).astype(np.float32)
         if reduction == "none" else 1.5)
    got = run_ex(inp, grad=g, z_loss=al, reduction=reduction, chunk=200)
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, wl.label_smoothing, reduction,
                                   np.asarray(g, dtype=np.float64), z_loss=al)
    tl, tg = TOL[dtype]
    valid = inp.labels != -100
    if reduction == "none":
        err = np.abs(got["loss"] - ref.loss).max() / np.abs(ref.loss[valid]).mean()
        assert np.all(got["loss"][~valid] == 0.0)
    else:
        err = abs(got["loss"][0] - ref.loss) / abs(ref.loss)
    ex, ew = rel_l2(got["dX"], ref.dX), rel_l2(got["dW"], ref.dW)
    print(f"[z-loss {al} {reduction} {dtype}] loss err {err:.2e}; dX {ex:.2e}; dW {ew:.2e}",
          flush=True)
    assert err <= tl and ex <= tg and ew <= tg
    assert rel_l2(got["lse"][valid], ref.lse[valid]) <= tl
    assert np.all(got["dX"][~valid] == 0.0)


def test_fused_none_is_unit_gradient():
    wl = wk.custom(520, 128, 3001, "bf16", 0.05, "uniform", ignore_frac=0.1, label_smoothing=0.05,
                   seed=73)
    inp = wk.draw(wl)
    got = run_ex(inp, split=False, reduction="none", z_loss=1e-4, chunk=128)
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, 0.05, "none", 1.0, z_loss=1e-4)
    valid = inp.labels != -100
    assert np.abs(got["loss"] - ref.loss).max() <= 2e-3 * np.abs(ref.loss[valid]).mean()
    assert rel_l2(got["dX"], ref.dX) <= 2e-2 and rel_l2(got["dW"], ref.dW) <= 2e-2


def test_ex_with_default_options_equals_plain_entry_points_bitwise():
    wl = wk.custom(900, 256, 4000, "bf16", 0.03, "zipf", 1.1, 0.03, 0.1, seed=75)
    inp = wk.draw(wl)
    for red in ("mean", "sum"):
        a = run(inp, chunk=300, reduction=red, split=True, grad=0.7)
        b = run_ex(inp, grad=0.7, reduction=red, chunk=300)
        assert a["loss"] == b["loss"][0]
        assert np.array_equal(a["dX"], b["dX"]) and np.array_equal(a["dW"], b["dW"])
        assert np.array_equal(a["lse"], b["lse"], equal_nan=True)


def test_none_flags_invalid_labels_with_nan():
    wl = wk.custom(200, 64, 500, "bf16", seed=77)
    inp = wk.draw(wl)
    inp.labels[[3, 50]] = [500, -7]  # outside [0, V), not ignore_index
    got = run_ex(inp, reduction="none", chunk=64)
    assert np.isnan(got["loss"][3]) and np.isnan(got["loss"][50])
    ok = np.ones(wl.N, bool)
    ok[[3, 50]] = False
    assert np.isfinite(got["loss"][ok]).all()


def test_full_size_zloss_none_sampled():
    # 4096 x 2048 x 32000 with z-loss and per-token gradients, against the
    # oracle on sampled rows of dX and dW and on every token's loss.
    wl = wk.WORKLOADS[2]
    inp = wk.draw(wl)
    al = 1e-4
    g = np.random.default_rng(9).uniform(-1.0, 1.0, wl.N).astype(np.float32)
    got = run_ex(inp, grad=g, z_loss=al, reduction="none", chunk=1024)
    loss, lse, _ = orc.forward(inp.X, inp.W, inp.labels, -100, wl.label_smoothing, "none",
                               z_loss=al)
    valid = inp.labels != -100
    assert np.abs(got["loss"] - loss).max() <= 2e-3 * np.abs(loss[valid]).mean()
    rows = np.random.default_rng(1).choice(wl.N, 64, replace=False)
    dx, _, _ = orc.dX_rows(inp.X, inp.W, inp.labels, rows, -100, wl.label_smoothing, "none",
                           g.astype(np.float64), z_loss=al)
    assert rel_l2(got["dX"][rows], dx) <= 2e-2
    vocab = np.random.default_rng(2).choice(wl.V, 64, replace=False)
    dw = orc.dW_rows(inp.X, inp.W, inp.labels, lse, vocab, -100, wl.label_smoothing, "none",
                     g.astype(np.float64), z_loss=al)
    assert rel_l2(got["dW"][vocab], dw) <= 2e-2


# ----------------------------------------------------- full-size workloads
def _golden(k):
    path = os.path.join(GOLDEN, f"oracle_config{k}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return np.load(path, allow_pickle=False)


_DRAWN = {}
_ORACLE = {}


def _draw_cached(k):
    if k not in _DRAWN:
        _DRAWN.clear()  # keep one full-size input in host memory at a time
        _DRAWN[k] = wk.draw(wk.WORKLOADS[k])
    return _DRAWN[k]


def tile_rows(n, tile=256, seed=0):
    """Rows to compare: in each tile of `tile` rows its first and last row
    and one drawn uniformly from the tile."""
    g = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, n, tile):
        t1 = min(n, t0 + tile)
        rows.update((t0, t1 - 1, int(g.integers(t0, t1))))
    return np.array(sorted(rows), dtype=np.int64)


def oracle_rows(k, inp, g):
    """The oracle's dX and dW rows for a full-size workload, computed now.

    4096 x 2048 x 32000: the whole oracle (every row).  Larger workloads:
    the rows of tile_rows over the tokens (dX) and the vocabulary (dW).  dW
    rows take every valid row's LSE from the stored oracle values (fp32: a
    relative error of at most |LSE| 2^-24 < 1e-6 in each softmax value, far
    below the bf16 bound); dX rows compute their own LSE in fp64."""
    if k in _ORACLE:
        return _ORACLE[k]
    wl = inp.workload
    eps = wl.label_smoothing
    if k == 2:
        ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, eps, "mean")
        assert abs(ref.loss - float(g["loss"])) <= 1e-12 * abs(ref.loss)
        out = dict(dx_idx=np.arange(wl.N), dx=ref.dX, dw_idx=np.arange(wl.V), dw=ref.dW,
                   whole=True)
    else:
        dx_idx = tile_rows(wl.N, seed=wl.seed)
        dw_idx = tile_rows(wl.V, seed=wl.seed + 1)
        dx, _, _ = orc.dX_rows(inp.X, inp.W, inp.labels, dx_idx, -100, eps, "mean")
        dw = orc.dW_rows(inp.X, inp.W, inp.labels, g["lse"], dw_idx, -100, eps, "mean")
        out = dict(dx_idx=dx_idx, dx=dx, dw_idx=dw_idx, dw=dw, whole=False)
    _ORACLE.clear()  # one workload's rows at a time
    _ORACLE[k] = out
    return out


# Every full-size workload at the benchmark's chunk, plus the chunk sweep at
# the headline shape and the token-chunk schedule there: all must agree with
# the same oracle values to the bf16 tolerance.
@pytest.mark.parametrize("k,chunk,schedule", [
    (2, 1024, "auto"), (3, 1024, "auto"), (3, 512, "auto"), (3, 256, "auto"),
    (3, 1024, "token"), (4, 1024, "auto"), (5, 1024, "auto")])
def test_full_size_workload(k, chunk, schedule):
    wl = wk.WORKLOADS[k]
    g = _golden(k)
    inp = _draw_cached(k)
    assert str(g["digest"]) == inp.digest(), "input generator drifted from the stored goldens"
    print(f"[{wl.name}] chunk {chunk} schedule {schedule}", flush=True)
    got = run(inp, chunk=chunk, schedule=schedule)
    check_full_size(k, inp, g, got, f"{wl.name} chunk {chunk} {schedule}")


def check_full_size(k, inp, g, got, label):
    """Full-size results against the oracle: the loss and every row's LSE
    (stored values), dX and dW on the rows of oracle_rows (whole tensors at
    4096 x 2048 x 32000), the rows stored with the goldens, and the dW
    column-sum invariant."""
    wl = inp.workload
    tl, tg = TOL[wl.dtype]
    ref = oracle_rows(k, inp, g)
    le = abs(got["loss"] - float(g["loss"])) / abs(float(g["loss"]))
    valid = inp.labels != -100
    e_lse = rel_l2(got["lse"][valid], g["lse"][valid])
    ex = rel_l2(got["dX"][ref["dx_idx"]], ref["dx"])
    ew = rel_l2(got["dW"][ref["dw_idx"]], ref["dw"])
    ex_s = rel_l2(got["dX"][g["dx_idx"]], g["dx"])
    ew_s = rel_l2(got["dW"][g["dw_idx"]], g["dw"])
    # the worst 256-row tile, by the relative L2 error of its compared rows
    def worst_tile(idx, a, b):
        tiles = idx // 256
        worst = 0.0
        for t in np.unique(tiles):
            sel = tiles == t
            worst = max(worst, rel_l2(a[sel], b[sel]))
        return worst
    wx = worst_tile(ref["dx_idx"], got["dX"][ref["dx_idx"]], ref["dx"])
    ww = worst_tile(ref["dw_idx"], got["dW"][ref["dw_idx"]], ref["dw"])
    col = np.linalg.norm(got["dW"].sum(axis=0, dtype=np.float64))
    fro = np.linalg.norm(got["dW"].astype(np.float64))
    what = "whole" if ref["whole"] else "rows"
    print(f"[{label}] loss {got['loss']:.7f} vs {float(g['loss']):.7f} rel {le:.2e}; "
          f"lse rel-L2 {e_lse:.2e}; dX {what} ({ref['dx_idx'].size}) {ex:.2e}, worst tile "
          f"{wx:.2e}; dW {what} ({ref['dw_idx'].size}) {ew:.2e}, worst tile {ww:.2e}; "
          f"stored rows dX {ex_s:.2e} dW {ew_s:.2e}; |sum_v dW|/|dW| {col / fro:.2e}",
          flush=True)
    parity_log.record(f"{label} [{what}: {ref['dx_idx'].size} dX, {ref['dw_idx'].size} dW rows]",
                      tl, tg, loss=le, lse=e_lse, dX=ex, dW=ew, dX_tile_max=wx, dW_tile_max=ww)
    assert le <= tl and e_lse <= tl
    assert ex <= tg and ew <= tg
    assert ex_s <= tg and ew_s <= tg
    assert np.all(got["dX"][~valid] == 0.0)
    assert col <= 1e-2 * fro  # rows of dZ sum to zero up to the bf16 rounding of dZ
    assert np.isfinite(got["dX"]).all() and np.isfinite(got["dW"]).all()


# ------------------------------------------- store-logits variant (6NVH)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_store_logits_against_oracle(dtype, reduction):
    # 700 tokens in chunks of 256 (the last one partial), ragged H and V,
    # smoothing, ignored rows and z-loss
    wl = wk.custom(700, 264 if dtype == "bf16" else 36, 5003, dtype, 0.05, "zipf", 1.1, 0.05, 0.1,
                   seed=91)
    inp = wk.draw(wl)
    al = 1e-3
    got = run_ex(inp, split=False, z_loss=al, reduction=reduction, chunk=200,
                 variant="store_logits")
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, wl.label_smoothing, reduction,
                                   1.0, z_loss=al)
    tl, tg = TOL[dtype]
    valid = inp.labels != -100
    if reduction == "none":
        err = np.abs(got["loss"] - ref.loss).max() / np.abs(ref.loss[valid]).mean()
        assert np.all(got["loss"][~valid] == 0.0)
    else:
        err = abs(got["loss"][0] - ref.loss) / abs(ref.loss)
    ex, ew = rel_l2(got["dX"], ref.dX), rel_l2(got["dW"], ref.dW)
    print(f"[store-logits {reduction} {dtype}] loss err {err:.2e}; dX {ex:.2e}; dW {ew:.2e}",
          flush=True)
    assert err <= tl and ex <= tg and ew <= tg
    assert np.all(got["dX"][~valid] == 0.0)
    # the loss comes from the same fp32 accumulators as the recompute path's
    rec = run_ex(inp, split=False, z_loss=al, reduction=reduction, chunk=200)
    assert np.allclose(got["loss"], rec["loss"], rtol=1e-6, atol=0.0, equal_nan=True)


def test_store_logits_chunk_of_ignored_rows_and_invalid_label():
    wl = wk.custom(600, 128, 3001, "bf16", 0.05, "uniform", ignore_frac=0.0, seed=93)
    inp = wk.draw(wl)
    inp.labels[256:512] = -100  # the whole second chunk
    got = run_ex(inp, split=False, chunk=256, variant="store_logits")
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, 0.0, "mean", 1.0)
    assert abs(got["loss"][0] - ref.loss) <= 2e-3 * abs(ref.loss)
    assert rel_l2(got["dX"], ref.dX) <= 2e-2 and rel_l2(got["dW"], ref.dW) <= 2e-2
    assert np.all(got["dX"][256:512] == 0.0)
    inp.labels[7] = 3001  # outside [0, V): NaN loss, the row's gradient is zero
    got = run_ex(inp, split=False, chunk=256, variant="store_logits")
    assert np.isnan(got["loss"][0]) and np.all(got["dX"][7] == 0.0)


@pytest.mark.parametrize("N,H,V", [(1, 8, 1), (5, 8, 2), (33, 8, 257), (257, 520, 300), (0, 8, 10)])
def test_store_logits_degenerate_shapes(N, H, V):
    inp = wk.draw(wk.custom(N, H, V, "bf16", 0.5, seed=95 + N))
    if N == 0:
        X = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
        _, W, _ = wk.to_torch(inp, "cuda")
        ws = fce.workspace_for(0, H, V, torch.bfloat16, variant="store_logits")
        loss = torch.full((1,), float("nan"), device="cuda")
        dW = torch.full((V, H), float("nan"), device="cuda")
        fce.fce_fused_fwd_bwd_ex(None, W, None, loss, None, dW, ws, variant="store_logits")
        torch.cuda.synchronize()
        assert loss.item() == 0.0 and torch.all(dW == 0).item()
        return
    got = run_ex(inp, split=False, chunk=64, variant="store_logits")
    ref = orc.linear_cross_entropy(inp.X, inp.W, inp.labels, -100, 0.0, "mean", 1.0)
    assert abs(got["loss"][0] - ref.loss) <= 2e-3 * max(abs(ref.loss), 1.0)
    # The kept logits are rounded to bf16 (relative error 2^-9) before
    # exp(z - LSE), so |error of dZ_ij| <= p_ij |z_ij| 2^-8 with the LSE from
    # fp32: an absolute floor that matters where dZ is ~0 (V = 1: p = 1).
    X64, W64 = inp.X.astype(np.float64), inp.W.astype(np.float64)
    zmax = np.abs(X64 @ W64.T).max()
    D = max(int((inp.labels != -100).sum()), 1)
    fx = 2.0 ** -8 * zmax * np.linalg.norm(W64, axis=1).max() * np.sqrt(N) / D
    fw = 2.0 ** -8 * zmax * np.linalg.norm(X64, axis=1).sum() / D
    assert np.linalg.norm(got["dX"] - ref.dX) <= 2e-2 * np.linalg.norm(ref.dX) + fx
    assert np.linalg.norm(got["dW"] - ref.dW) <= 2e-2 * np.linalg.norm(ref.dW) + fw


# The headline shape in one chunk (the whole 8192 x 128256 logits kept) and
# in chunks of 1024, and the 4096 x 2048 x 32000 workload.
@pytest.mark.parametrize("k,chunk", [(2, 1024), (3, 1024), (3, 8192), (4, 2048), (5, 1024)])
def test_store_logits_full_size(k, chunk):
    wl = wk.WORKLOADS[k]
    g = _golden(k)
    inp = _draw_cached(k)
    assert str(g["digest"]) == inp.digest(), "input generator drifted from the stored goldens"
    print(f"[{wl.name}] store-logits chunk {chunk}", flush=True)
    got = run_ex(inp, split=False, chunk=chunk, variant="store_logits")
    got["loss"] = float(got["loss"][0])
    # the LSE stays in the workspace; take it from the forward entry point
    got["lse"] = run_ex_lse(inp)
    check_full_size(k, inp, g, got, f"{wl.name} store-logits chunk {chunk}")


@pytest.mark.parametrize("k", [4, 5])
def test_filtered_full_size(k):
    # the filtered variant at the two largest workloads (label smoothing at
    # 16384 x 3584 x 152064): against the stored oracle values
    wl = wk.WORKLOADS[k]
    g = _golden(k)
    inp = _draw_cached(k)
    assert str(g["digest"]) == inp.digest(), "input generator drifted from the stored goldens"
    X, W, y = wk.to_torch(inp, "cuda")
    ws = fce.workspace_for(wl.N, wl.H, wl.V, X.dtype, variant="filtered",
                           label_smoothing=wl.label_smoothing)
    loss = torch.empty(1, device="cuda")
    dX = torch.empty((wl.N, wl.H), device="cuda")
    dW = torch.empty((wl.V, wl.H), device="cuda")
    fce.fce_fused_fwd_bwd_ex(X, W, y, loss, dX, dW, ws, variant="filtered",
                             label_smoothing=wl.label_smoothing)
    torch.cuda.synchronize()
    kept, total = fce.fce_get_filter_stats(ws)
    print(f"[{wl.name} filtered] kept {kept}/{total}", flush=True)
    got = dict(loss=loss.item(), lse=run_ex_lse(inp), dX=dX.cpu().numpy(), dW=dW.cpu().numpy())
    check_full_size(k, inp, g, got, f"{wl.name} filtered")


def run_ex_lse(inp):
    X, W, y = wk.to_torch(inp, "cuda")
    wl = inp.workload
    ws = fce.workspace_for(wl.N, wl.H, wl.V, X.dtype)
    loss = torch.empty(1, device="cuda")
    lse = torch.empty(wl.N, device="cuda")
    fce.fce_forward(X, W, y, loss, lse, ws, -100, wl.label_smoothing, "mean", 1024, "auto")
    torch.cuda.synchronize()
    return lse.cpu().numpy()
