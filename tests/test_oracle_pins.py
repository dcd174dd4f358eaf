"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each check is independent of the oracle's own formulas: closed forms,
invariants, central finite differences, and torch's fp64 cross_entropy with
autograd on small shapes.  ``test_planted_mistakes_are_caught`` plants
plausible mistakes in the oracle (on the CPU) and requires some pin to fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle.fce_oracle as orc

RNG = np.random.default_rng(12345)


def _case(N, H, V, ignore=0, seed=0, xs=1.0, ws=0.5):
    g = np.random.default_rng(seed)
    X = g.standard_normal((N, H)) * xs
    W = g.standard_normal((V, H)) * ws
    y = g.integers(0, V, size=N)
    if ignore:
        y[g.choice(N, size=ignore, replace=False)] = -100
    return X, W, y


# --------------------------------------------------------------- closed forms
def check_zero_weights_give_log_V():
    # W = 0: every logit is 0, softmax is uniform, loss = log V for any
    # smoothing and mask ([LLMS] "The Vocabulary Memory Wall" loss with z = 0).
    for V, eps in [(7, 0.0), (50, 0.1), (1000, 0.3)]:
        X, _, y = _case(9, 5, V, ignore=3, seed=V)
        W = np.zeros((V, 5))
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps)
        assert abs(r.loss - math.log(V)) < 1e-12, (V, eps, r.loss)
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, reduction="sum")
        assert abs(r.loss - 6 * math.log(V)) < 1e-10


def check_two_class_closed_form():
    # N = 1, H = 1, V = 2, x = 1, W = (a, b), label 0: the loss is the
    # cross-entropy between target (1 - eps/2, eps/2) and the logistic
    # probabilities, i.e. (1-eps/2) softplus(b-a) + (eps/2) softplus(a-b);
    # its derivative wrt (a, b) is (sigmoid(a-b) - 1 + eps/2, sigmoid(b-a) - eps/2).
    def softplus(t):
        return math.log1p(math.exp(-abs(t))) + max(t, 0.0)

    def sigmoid(t):
        return 1.0 / (1.0 + math.exp(-t))

    for a, b, eps in [(0.3, -1.2, 0.0), (2.0, 5.0, 0.0), (-1.0, 0.7, 0.2), (4.0, 4.0, 0.5)]:
        X = np.array([[1.0]])
        W = np.array([[a], [b]])
        r = orc.linear_cross_entropy(X, W, np.array([0]), label_smoothing=eps)
        want = (1 - eps / 2) * softplus(b - a) + (eps / 2) * softplus(a - b)
        assert abs(r.loss - want) < 1e-13, (a, b, eps)
        ga = sigmoid(a - b) - (1 - eps / 2)
        gb = sigmoid(b - a) - eps / 2
        assert np.allclose(r.dW[:, 0], [ga, gb], atol=1e-14)
        assert abs(r.dX[0, 0] - (ga * a + gb * b)) < 1e-13


def check_single_class_is_zero():
    # V = 1: softmax is 1 at the only class, loss and gradients vanish.
    X, W, _ = _case(6, 4, 1, seed=3)
    y = np.zeros(6, dtype=np.int64)
    for eps in (0.0, 0.25):
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps)
        assert abs(r.loss) < 1e-14
        assert np.abs(r.dX).max() < 1e-14 and np.abs(r.dW).max() < 1e-14


def check_uniform_logits_closed_form():
    # X = 0: every logit is 0, so p = 1/V; dZ_ij = (1/V - q_ij)/D, dW = dZ^T X = 0
    # and dX_i = (1-eps) (mean_j W_j - W_{y_i}) / D.
    V, H, N = 11, 4, 7
    _, W, y = _case(N, H, V, ignore=2, seed=5)
    X = np.zeros((N, H))
    eps = 0.2
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps)
    D = 5.0
    assert abs(r.loss - math.log(V)) < 1e-13
    assert np.abs(r.dW).max() == 0.0
    for i in range(N):
        if y[i] == -100:
            assert np.all(r.dX[i] == 0.0)
        else:
            want = (1 - eps) * (W.mean(axis=0) - W[y[i]]) / D
            assert np.allclose(r.dX[i], want, atol=1e-14)


# ------------------------------------------------------------ library routine
def check_matches_torch_cross_entropy():
    # torch's F.cross_entropy on materialised logits, fp64 on the CPU, with
    # autograd: the unfused pipeline of [LLMS] "The Standard Execution
    # Pipeline" and the per-chunk call of [CCE]'s chunked module.
    cases = [(64, 32, 512, 6, 0.0, "mean"), (40, 16, 300, 0, 0.1, "mean"),
             (33, 8, 129, 5, 0.3, "sum"), (17, 24, 64, 16, 0.05, "mean")]
    for n, (N, H, V, ign, eps, red) in enumerate(cases):
        X, W, y = _case(N, H, V, ignore=ign, seed=100 + n)
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, reduction=red, grad_loss=1.7)
        Xt = torch.tensor(X, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        L = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(y), ignore_index=-100,
                                              label_smoothing=eps, reduction=red)
        (L * 1.7).backward()
        assert abs(r.loss - L.item()) <= 1e-12 * max(1.0, abs(L.item())), (n, r.loss, L.item())
        assert np.allclose(r.dX, Xt.grad.numpy(), rtol=1e-10, atol=1e-13), n
        assert np.allclose(r.dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-13), n


# ------------------------------------------------------------- brute force
def check_finite_differences():
    # Central differences of the oracle's own loss, fp64, tiny shapes: the
    # gradient must be the derivative of the loss.
    h = 1e-6
    for seed, (N, H, V, ign, eps, red) in enumerate([(8, 8, 16, 2, 0.1, "mean"), (5, 3, 9, 0, 0.0, "sum"),
                                                     (6, 4, 12, 1, 0.3, "mean")]):
        X, W, y = _case(N, H, V, ignore=ign, seed=200 + seed)
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, reduction=red, grad_loss=0.8)

        def L(X_, W_):
            return 0.8 * orc.linear_cross_entropy(X_, W_, y, label_smoothing=eps, reduction=red).loss

        for (i, k) in [(a, b) for a in range(N) for b in range(H)]:
            Xp = X.copy(); Xp[i, k] += h
            Xm = X.copy(); Xm[i, k] -= h
            fd = (L(Xp, W) - L(Xm, W)) / (2 * h)
            assert abs(fd - r.dX[i, k]) < 1e-7, ("dX", seed, i, k, fd, r.dX[i, k])
        for (v, k) in [(a, b) for a in range(V) for b in range(H)]:
            Wp = W.copy(); Wp[v, k] += h
            Wm = W.copy(); Wm[v, k] -= h
            fd = (L(X, Wp) - L(X, Wm)) / (2 * h)
            assert abs(fd - r.dW[v, k]) < 1e-7, ("dW", seed, v, k, fd, r.dW[v, k])


# ----------------------------------------------------------------- invariants
def check_gradient_rows_sum_to_zero():
    # Each row of dZ sums to 0 (softmax and q both sum to 1), hence
    # sum_v dW[v, :] = 0 ([LLMS] step 3's gradient).
    X, W, y = _case(30, 12, 77, ignore=4, seed=7)
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=0.15)
    assert np.abs(r.dW.sum(axis=0)).max() < 1e-14 * 77 * 30
    Z = orc.logits(X[y != -100], W)
    lse = orc.log_sum_exp(Z)
    dZ = orc.dlogits(Z, lse, y[y != -100], 0.15, 1.0)
    assert np.abs(dZ.sum(axis=1)).max() < 1e-14


def check_ignored_rows_are_inert():
    # label == ignore_index: zero dX row; changing that X row changes
    # neither the loss nor dW ([LLMS] "Numerical Considerations" item 2).
    X, W, y = _case(20, 6, 40, ignore=5, seed=9)
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=0.1)
    ign = y == -100
    assert np.all(r.dX[ign] == 0.0)
    X2 = X.copy()
    X2[ign] = 1e3 * RNG.standard_normal((ign.sum(), 6))
    r2 = orc.linear_cross_entropy(X2, W, y, label_smoothing=0.1)
    assert r2.loss == r.loss
    assert np.array_equal(r2.dW, r.dW)


def check_shift_invariance():
    # W -> W + 1 u^T adds x_i.u to every logit of row i: LSE and all logits
    # shift together, so the loss, dZ, dX and dW are unchanged ([CCE]
    # "Online Log-Sum-Exp": LSE(z) = m + log sum exp(z - m) for any m).
    X, W, y = _case(25, 7, 60, ignore=3, seed=11)
    u = RNG.standard_normal(7)
    a = orc.linear_cross_entropy(X, W, y, label_smoothing=0.2)
    b = orc.linear_cross_entropy(X, W + u[None, :], y, label_smoothing=0.2)
    assert abs(a.loss - b.loss) < 1e-12
    assert np.allclose(a.dX, b.dX, atol=1e-13)
    assert np.allclose(a.dW, b.dW, atol=1e-13)


def check_large_logits_stay_finite():
    # Logits far above exp's fp32 overflow point ([CCE] "Numerical
    # Stability": exp overflows for x > 88.7) still give finite results that
    # agree with the logistic closed form in the two-class case.
    X, W, y = _case(16, 8, 50, seed=13, xs=100.0)
    r = orc.linear_cross_entropy(X, W, y)
    assert np.isfinite(r.loss) and np.isfinite(r.dX).all() and np.isfinite(r.dW).all()
    r2 = orc.linear_cross_entropy(np.array([[1.0]]), np.array([[800.0], [-300.0]]), np.array([1]))
    assert abs(r2.loss - 1100.0) < 1e-9


def check_all_ignored_gives_zero():
    # D = max(N_valid, 1) ([CCE] chunked module's final division): with
    # every row ignored the loss and gradients are 0, not NaN.
    X, W, _ = _case(5, 3, 10, seed=15)
    y = np.full(5, -100)
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=0.1)
    assert r.loss == 0.0 and r.n_valid == 0
    assert not r.dX.any() and not r.dW.any()


def check_row_block_invariance():
    # Row blocks only bound memory: per-row results agree to fp64 rounding
    # (BLAS may pick a different kernel for a different block height).
    X, W, y = _case(37, 9, 101, ignore=6, seed=17)
    ref = orc.linear_cross_entropy(X, W, y, label_smoothing=0.1, row_block=1000)
    for rb in (1, 7, 16):
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=0.1, row_block=rb)
        assert abs(r.loss - ref.loss) < 1e-13
        assert np.allclose(r.dX, ref.dX, rtol=1e-13, atol=1e-16)
        assert np.allclose(r.dW, ref.dW, rtol=1e-13, atol=1e-16)


# ------------------------------------------------- z-loss and reduction none
def check_zloss_zero_weights():
    # W = 0: LSE = log V in every row, so l_i = log V + alpha log^2 V
    # ([LLMS] "Numerical Considerations" item 3: L_z = alpha log^2 sum exp z).
    for V, eps, a in [(7, 0.0, 1e-2), (50, 0.1, 0.3), (1000, 0.3, 1e-4)]:
        X, _, y = _case(9, 5, V, ignore=3, seed=V + 1)
        W = np.zeros((V, 5))
        want = math.log(V) + a * math.log(V) ** 2
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, z_loss=a)
        assert abs(r.loss - want) < 1e-12, (V, eps, a, r.loss, want)
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, z_loss=a, reduction="none")
        assert np.allclose(r.loss[y != -100], want, atol=1e-12) and np.all(r.loss[y == -100] == 0)


def check_zloss_two_class_closed_form():
    # N = H = 1, V = 2, x = 1, W = (a, b), label 0, no smoothing:
    # l = softplus(b - a) + alpha s^2 with s = log(e^a + e^b); then
    # dl/da = sigmoid(a - b) (1 + 2 alpha s) - 1 and dl/db = sigmoid(b - a) (1 + 2 alpha s).
    def sigmoid(t):
        return 1.0 / (1.0 + math.exp(-t))

    for a, b, al in [(0.3, -1.2, 0.1), (2.0, 5.0, 0.01), (-1.0, 0.7, 1.0)]:
        s = max(a, b) + math.log(math.exp(a - max(a, b)) + math.exp(b - max(a, b)))
        want = s - a + al * s * s
        r = orc.linear_cross_entropy(np.array([[1.0]]), np.array([[a], [b]]), np.array([0]),
                                     z_loss=al)
        assert abs(r.loss - want) < 1e-13, (a, b, al)
        ga = sigmoid(a - b) * (1 + 2 * al * s) - 1
        gb = sigmoid(b - a) * (1 + 2 * al * s)
        assert np.allclose(r.dW[:, 0], [ga, gb], atol=1e-13)


def _torch_reference(X, W, y, eps, red, g, al):
    """torch fp64 autograd of F.cross_entropy(reduction="none") plus
    alpha logsumexp^2 on the valid rows, reduced as asked."""
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    Z = Xt @ Wt.T
    yt = torch.tensor(y)
    ce = torch.nn.functional.cross_entropy(Z, yt, ignore_index=-100, label_smoothing=eps,
                                           reduction="none")
    valid = (yt != -100).double()
    per = ce + al * torch.logsumexp(Z, dim=1) ** 2 * valid
    if red == "none":
        L = per
        (per * torch.tensor(g)).sum().backward()
    else:
        L = per.sum() / (max(float(valid.sum()), 1.0) if red == "mean" else 1.0)
        (L * g).backward()
    return L.detach().numpy(), Xt.grad.numpy(), Wt.grad.numpy()


def check_zloss_and_none_match_torch():
    cases = [(40, 16, 300, 5, 0.1, "mean", 0.05), (33, 8, 129, 4, 0.0, "sum", 0.2),
             (29, 12, 200, 6, 0.2, "none", 0.1), (17, 24, 64, 3, 0.0, "none", 0.0)]
    for n, (N, H, V, ign, eps, red, al) in enumerate(cases):
        X, W, y = _case(N, H, V, ignore=ign, seed=400 + n)
        g = np.random.default_rng(n).uniform(-2.0, 2.0, N) if red == "none" else 1.3
        r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, reduction=red, grad_loss=g,
                                     z_loss=al)
        L, dX, dW = _torch_reference(X, W, y, eps, red, g, al)
        assert np.allclose(r.loss, L, rtol=1e-12, atol=1e-13), n
        assert np.allclose(r.dX, dX, rtol=1e-10, atol=1e-13), n
        assert np.allclose(r.dW, dW, rtol=1e-10, atol=1e-13), n


def check_zloss_none_finite_differences():
    # d/dtheta of sum_i g_i l_i with per-row weights, z-loss and smoothing.
    h = 1e-6
    N, H, V = 6, 4, 11
    X, W, y = _case(N, H, V, ignore=1, seed=500)
    g = np.random.default_rng(5).uniform(-1.5, 1.5, N)
    al, eps = 0.2, 0.1
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, reduction="none", grad_loss=g,
                                 z_loss=al)

    def L(X_, W_):
        l = orc.linear_cross_entropy(X_, W_, y, label_smoothing=eps, reduction="none",
                                     z_loss=al).loss
        return float((g * l).sum())

    for i in range(N):
        for k in range(H):
            Xp = X.copy(); Xp[i, k] += h
            Xm = X.copy(); Xm[i, k] -= h
            assert abs((L(Xp, W) - L(Xm, W)) / (2 * h) - r.dX[i, k]) < 1e-7, ("dX", i, k)
    for v in range(V):
        for k in range(H):
            Wp = W.copy(); Wp[v, k] += h
            Wm = W.copy(); Wm[v, k] -= h
            assert abs((L(X, Wp) - L(X, Wm)) / (2 * h) - r.dW[v, k]) < 1e-7, ("dW", v, k)


def check_reductions_agree():
    # none summed = sum; mean = sum / N_valid; a constant per-row gradient c
    # under "none" gives c times the "sum" gradients.
    X, W, y = _case(31, 7, 90, ignore=4, seed=600)
    kw = dict(label_smoothing=0.1, z_loss=0.03)
    none = orc.linear_cross_entropy(X, W, y, reduction="none", grad_loss=np.full(31, 0.7), **kw)
    s = orc.linear_cross_entropy(X, W, y, reduction="sum", grad_loss=0.7, **kw)
    m = orc.linear_cross_entropy(X, W, y, reduction="mean", **kw)
    assert abs(none.loss.sum() - s.loss) < 1e-12 * abs(s.loss)
    assert abs(m.loss - s.loss / 27) < 1e-13
    assert np.allclose(none.dX, s.dX, atol=1e-15) and np.allclose(none.dW, s.dW, atol=1e-15)


def check_logits_path_matches_torch():
    # Loss and dZ on given logits ([L27] "Trick 1"): torch autograd on Z.
    for n, (N, V, ign, eps, red, al) in enumerate([(20, 50, 3, 0.1, "mean", 0.01),
                                                   (15, 33, 0, 0.0, "none", 0.2),
                                                   (9, 7, 2, 0.3, "sum", 0.0)]):
        rng = np.random.default_rng(700 + n)
        Z = rng.standard_normal((N, V)) * 3.0
        y = rng.integers(0, V, N)
        y[rng.choice(N, ign, replace=False)] = -100
        g = rng.uniform(-1, 1, N) if red == "none" else 0.9
        loss, lse, dZ = orc.softmax_ce_on_logits(Z, y, label_smoothing=eps, reduction=red,
                                                 grad_loss=g, z_loss=al)
        Zt = torch.tensor(Z, requires_grad=True)
        yt = torch.tensor(y)
        ce = torch.nn.functional.cross_entropy(Zt, yt, ignore_index=-100, label_smoothing=eps,
                                               reduction="none")
        valid = (yt != -100).double()
        per = ce + al * torch.logsumexp(Zt, dim=1) ** 2 * valid
        if red == "none":
            (per * torch.tensor(g)).sum().backward()
            L = per.detach().numpy()
        else:
            Lt = per.sum() / (max(float(valid.sum()), 1.0) if red == "mean" else 1.0)
            (Lt * g).backward()
            L = Lt.item()
        assert np.allclose(loss, L, rtol=1e-12, atol=1e-13), n
        assert np.allclose(dZ, Zt.grad.numpy(), rtol=1e-10, atol=1e-14), n
        v = y != -100
        assert np.allclose(lse[v], torch.logsumexp(torch.tensor(Z), 1).numpy()[v], atol=1e-13)


# ------------------------------------------------------- gradient filtering
def check_filter_threshold_zero_keeps_everything():
    # every softmax value is >= 0: nothing is dropped, the gradients are exact
    X, W, y = _case(300, 6, 530, ignore=20, seed=41)
    f = orc.filtered_linear_cross_entropy(X, W, y, label_smoothing=0.1, z_loss=1e-2, tile=64,
                                          threshold=0.0)
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=0.1, z_loss=1e-2)
    assert f.keep.all() and f.keep.shape == (5, 9)
    assert np.allclose(f.result.dX, r.dX, atol=1e-14) and np.allclose(f.result.dW, r.dW, atol=1e-14)
    assert f.result.loss == r.loss


def _filter_brute_force(X, W, y, eps, al, tile, thr, ignore=-100):
    # the block rule written out element by element with math.* (independent
    # of the oracle's vectorised form)
    N, H = X.shape
    V = W.shape[0]
    rows = [i for i in range(N) if y[i] != ignore]
    D = max(len(rows), 1)
    z = [[math.fsum(X[i, k] * W[j, k] for k in range(H)) for j in range(V)] for i in range(N)]
    lse = {}
    for i in rows:
        m = max(z[i])
        lse[i] = m + math.log(math.fsum(math.exp(v - m) for v in z[i]))
    p = {(i, j): math.exp(z[i][j] - lse[i]) for i in rows for j in range(V)}
    kept = {}
    for I in range(-(-N // tile)):
        for J in range(-(-V // tile)):
            rr = [i for i in rows if I * tile <= i < (I + 1) * tile]
            cc = range(J * tile, min(V, (J + 1) * tile))
            kept[I, J] = any(y[i] in cc for i in rr) or any(p[i, j] >= thr for i in rr for j in cc)
    dz = np.zeros((N, V))
    for i in rows:
        for j in range(V):
            if kept[i // tile, j // tile]:
                q = (1 - eps) * (j == y[i]) + eps / V
                dz[i, j] = (p[i, j] * (1 + 2 * al * lse[i]) - q) / D
    dX = [[math.fsum(dz[i, j] * W[j, k] for j in range(V)) for k in range(H)] for i in range(N)]
    dW = [[math.fsum(dz[i, j] * X[i, k] for i in range(N)) for k in range(H)] for j in range(V)]
    return kept, np.array(dX), np.array(dW)


def check_filter_brute_force_tiny():
    X, W, y = _case(7, 3, 9, ignore=2, seed=43, ws=0.9)
    for thr in (0.08, 0.2):
        f = orc.filtered_linear_cross_entropy(X, W, y, label_smoothing=0.1, z_loss=0.05, tile=2,
                                              threshold=thr)
        kept, dX, dW = _filter_brute_force(X, W, y, 0.1, 0.05, 2, thr)
        assert {k: bool(f.keep[k]) for k in kept} == kept, thr
        assert not all(kept.values()) and any(kept.values())
        assert np.allclose(f.result.dX, dX, atol=1e-13) and np.allclose(f.result.dW, dW, atol=1e-13)


def check_filter_dropped_entries_are_bounded():
    # an entry of a dropped block is (p (1 + 2 alpha LSE) - eps/V) s with
    # p < threshold: its magnitude is below s max(threshold (1 + 2 alpha LSE), eps/V)
    # labels in the first block of columns, a flat softmax over V = 2000
    X, W, y = _case(200, 8, 2000, ignore=10, seed=47, ws=0.2)
    y = np.where(y == -100, y, y % 16)
    eps, al, thr = 0.1, 0.02, 2.0 ** -9
    f = orc.filtered_linear_cross_entropy(X, W, y, label_smoothing=eps, z_loss=al, tile=16,
                                          threshold=thr)
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=eps, z_loss=al)
    v = y != -100
    Z = X[v] @ W.T
    lse = r.lse[v]
    full = orc.dlogits(Z, lse, y[v], eps, 1.0 / v.sum(), al)
    diff = np.abs(full - f.dZ[v])
    bound = np.maximum(thr * (1 + 2 * al * lse), eps / 2000) / v.sum()
    assert (diff <= bound[:, None] + 1e-17).all()
    assert (~f.keep).any()  # something was dropped


def check_filter_infinite_threshold_keeps_label_blocks_only():
    X, W, y = _case(260, 5, 1000, ignore=30, seed=53)
    f = orc.filtered_linear_cross_entropy(X, W, y, tile=64, threshold=np.inf)
    want = np.zeros_like(f.keep)
    for i in np.nonzero(y != -100)[0]:
        want[i // 64, y[i] // 64] = True
    assert np.array_equal(f.keep, want)


CHECKS = [check_zero_weights_give_log_V, check_two_class_closed_form, check_single_class_is_zero,
          check_uniform_logits_closed_form, check_matches_torch_cross_entropy,
          check_finite_differences, check_gradient_rows_sum_to_zero, check_ignored_rows_are_inert,
          check_shift_invariance, check_large_logits_stay_finite, check_all_ignored_gives_zero,
          check_row_block_invariance, check_zloss_zero_weights, check_zloss_two_class_closed_form,
          check_zloss_and_none_match_torch, check_zloss_none_finite_differences,
          check_reductions_agree, check_logits_path_matches_torch,
          check_filter_threshold_zero_keeps_everything, check_filter_brute_force_tiny,
          check_filter_dropped_entries_are_bounded,
          check_filter_infinite_threshold_keeps_label_blocks_only]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__[6:] for c in CHECKS])
def test_pin(check):
    check()


def test_out_of_range_label_raises():
    X, W, y = _case(4, 3, 10, seed=19)
    y[2] = 10
    with pytest.raises(ValueError):
        orc.linear_cross_entropy(X, W, y)
    y[2] = -1
    with pytest.raises(ValueError):
        orc.linear_cross_entropy(X, W, y)


def test_sampled_rows_match_full():
    # The sampled entry points used at full workload sizes agree with the
    # full computation (they are built from the same pinned steps).
    X, W, y = _case(50, 10, 200, ignore=5, seed=21)
    r = orc.linear_cross_entropy(X, W, y, label_smoothing=0.1, grad_loss=2.0)
    rows = np.array([0, 3, 17, 49] + list(np.nonzero(y == -100)[0][:2]))
    dx, lse, terms = orc.dX_rows(X, W, y, rows, label_smoothing=0.1, grad_loss=2.0)
    assert np.allclose(dx, r.dX[rows], atol=1e-15)
    v = np.array([0, 5, 199, int(y[0])])
    dw = orc.dW_rows(X, W, y, r.lse, v, label_smoothing=0.1, grad_loss=2.0)
    assert np.allclose(dw, r.dW[v], atol=1e-14)
    loss, lse_f, nv = orc.forward(X, W, y, label_smoothing=0.1)
    assert abs(loss - r.loss) < 1e-13 and nv == r.n_valid
    # the same with z-loss and per-row gradients (reduction "none")
    g = np.random.default_rng(3).uniform(-1, 1, 50)
    kw = dict(label_smoothing=0.1, reduction="none", z_loss=0.05)
    r = orc.linear_cross_entropy(X, W, y, grad_loss=g, **kw)
    dx, lse, terms = orc.dX_rows(X, W, y, rows, grad_loss=g, **kw)
    assert np.allclose(dx, r.dX[rows], atol=1e-15)
    assert np.allclose(terms, r.loss[rows], atol=1e-14)
    dw = orc.dW_rows(X, W, y, r.lse, v, grad_loss=g, **kw)
    assert np.allclose(dw, r.dW[v], atol=1e-14)
    loss, _, _ = orc.forward(X, W, y, **{k: kw[k] for k in kw})
    assert np.allclose(loss, r.loss, atol=1e-14)


# ----------------------------------------------------------- planted mistakes
def _mutants():
    """Plausible mistakes, each planted into a copy of the oracle's steps."""
    base_tl, base_dl, base_den = orc.token_losses, orc.dlogits, orc.denominator
    base_lse = orc.log_sum_exp

    def tl_drop_smooth(Z, lse, y, eps, z_loss=0.0):
        return base_tl(Z, lse, y, 0.0, z_loss)

    def tl_sign(Z, lse, y, eps, z_loss=0.0):
        return -base_tl(Z, lse, y, eps, z_loss)

    def tl_wrong_index(Z, lse, y, eps, z_loss=0.0):
        return base_tl(Z, lse, (y + 1) % Z.shape[1], eps, z_loss)

    def tl_drop_zloss(Z, lse, y, eps, z_loss=0.0):
        return base_tl(Z, lse, y, eps, 0.0)

    def tl_zloss_not_squared(Z, lse, y, eps, z_loss=0.0):
        return base_tl(Z, lse, y, eps, 0.0) + z_loss * lse

    def dl_drop_smooth(Z, lse, y, eps, scale, z_loss=0.0):
        return base_dl(Z, lse, y, 0.0, scale, z_loss)

    def dl_no_onehot_scale(Z, lse, y, eps, scale, z_loss=0.0):
        P = np.exp(Z - lse[:, None]) * (1.0 + 2.0 * z_loss * lse)[:, None]
        P[np.arange(Z.shape[0]), y] -= 1.0
        sc = np.asarray(scale)
        return (P - eps / Z.shape[1]) * (sc[:, None] if sc.ndim else sc)

    def dl_zloss_half(Z, lse, y, eps, scale, z_loss=0.0):
        return base_dl(Z, lse, y, eps, scale, 0.5 * z_loss)

    def dl_zloss_on_target(Z, lse, y, eps, scale, z_loss=0.0):
        # z-loss factor applied to (p - q) instead of p
        d = base_dl(Z, lse, y, eps, 1.0, 0.0) * (1.0 + 2.0 * z_loss * lse)[:, None]
        sc = np.asarray(scale)
        return d * (sc[:, None] if sc.ndim else sc)

    def rs_ignore_rows(grad_loss, n_rows, D, reduction):
        g = np.asarray(grad_loss, dtype=np.float64)
        return np.full(n_rows, float(g.mean()) / D)

    def den_all_rows(n_valid, reduction):
        return base_den(n_valid + 1, reduction)

    def lse_no_max(Z):
        return np.log(np.exp(Z).sum(axis=1))

    def lse_drop_max(Z):
        return np.log(np.exp(Z - Z.max(axis=1)[:, None]).sum(axis=1))

    def logits_transposed_bad(X, W):
        return X @ W.T * 1.0000001

    base_flt = orc.filtered_linear_cross_entropy

    def _refilter(f, X, W, tile, keep):
        # the same result with another kept-block set
        dZ = f.dZ.copy()
        for I in range(keep.shape[0]):
            for J in range(keep.shape[1]):
                if not keep[I, J]:
                    dZ[I * tile:(I + 1) * tile, J * tile:(J + 1) * tile] = 0.0
        res = orc.OracleResult(f.result.loss, f.result.lse, dZ @ np.asarray(W, float),
                               dZ.T @ np.asarray(X, float), f.result.n_valid)
        return orc.FilteredResult(res, keep, dZ)

    def flt_drops_label_blocks(X, W, labels, ignore_index=-100, label_smoothing=0.0,
                               reduction="mean", grad_loss=1.0, z_loss=0.0, tile=256,
                               threshold=2.0 ** -12):
        # the target term's block is dropped like any other
        f = base_flt(X, W, labels, ignore_index, label_smoothing, reduction, grad_loss, z_loss,
                     tile, 0.0)
        y = np.asarray(labels)
        V = np.asarray(W).shape[0]
        v = y != ignore_index
        Z = np.asarray(X, float)[v] @ np.asarray(W, float).T
        P = np.zeros((len(y), V))
        P[v] = np.exp(Z - f.result.lse[v][:, None])
        keep = np.zeros_like(f.keep)
        for I in range(keep.shape[0]):
            for J in range(keep.shape[1]):
                keep[I, J] = (P[I * tile:(I + 1) * tile, J * tile:(J + 1) * tile] >= threshold).any()
        return _refilter(f, X, W, tile, keep)

    def flt_shifted_blocks(X, W, labels, ignore_index=-100, label_smoothing=0.0,
                           reduction="mean", grad_loss=1.0, z_loss=0.0, tile=256,
                           threshold=2.0 ** -12):
        # block flags computed one token too early (an off-by-one row index)
        f = base_flt(X, W, labels, ignore_index, label_smoothing, reduction, grad_loss, z_loss,
                     tile, threshold)
        g = base_flt(np.roll(np.asarray(X), -1, axis=0), W, np.roll(np.asarray(labels), -1),
                     ignore_index, label_smoothing, reduction, grad_loss, z_loss, tile, threshold)
        return _refilter(f, X, W, tile, g.keep)

    return [("token_losses", tl_drop_smooth), ("token_losses", tl_sign),
            ("token_losses", tl_wrong_index), ("token_losses", tl_drop_zloss),
            ("token_losses", tl_zloss_not_squared), ("dlogits", dl_drop_smooth),
            ("dlogits", dl_no_onehot_scale), ("dlogits", dl_zloss_half),
            ("dlogits", dl_zloss_on_target), ("row_scales", rs_ignore_rows),
            ("denominator", den_all_rows),
            ("log_sum_exp", lse_no_max), ("log_sum_exp", lse_drop_max),
            ("logits", logits_transposed_bad),
            ("filtered_linear_cross_entropy", flt_drops_label_blocks),
            ("filtered_linear_cross_entropy", flt_shifted_blocks)]


@pytest.mark.parametrize("name,fn", _mutants(), ids=lambda m: getattr(m, "__name__", str(m)))
def test_planted_mistakes_are_caught(monkeypatch, name, fn):
    monkeypatch.setattr(orc, name, fn)
    failures = 0
    with np.errstate(all="ignore"):
        for check in CHECKS:
            try:
                check()
            except (AssertionError, FloatingPointError, ValueError, OverflowError):
                failures += 1
    assert failures > 0, f"no pin catches the planted mistake in {name}"
