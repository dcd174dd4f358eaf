"""Plain fp64 CPU oracle for linear cross-entropy (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

It computes the plain definition, in float64, with every logit row
materialised (rows are processed in blocks only to bound host memory; the
block size does not change the arithmetic order within a row).

Sources (cited by page title and section):
  [LLMS]  "Chunked and Fused Cross-Entropy: How Online Logit Tiling Slashes
          Large-Vocabulary VRAM Bottlenecks in LLM Training" (llms.blog)
  [CCE]   "Cut Cross-Entropy: Memory-Efficient Large-Vocab LLM Guide"
          (aifetchly blog)
  [L27]   "Fused cross-entropy -- the memory kernel" (lesson 27)

Definitions used (notation of [LLMS]):
  Z = X W^T                                    [LLMS, "The Vocabulary Memory Wall", first equation]
  m_i = max_j z_ij, d_i = sum_j exp(z_ij - m_i),
  LSE_i = m_i + log d_i                        [LLMS, "Mathematical Mechanics", step 2;
                                                CCE, "Numerical Stability and Maximum Subtraction"]
  l_i = LSE_i - z_{i,y_i}                      [LLMS step 2; CCE "Online Log-Sum-Exp"]
  dL/dz_ij = (softmax_ij - [j = y_i]) / N      [LLMS step 3; L27 "The gradient that makes fusion trivial"]
  dX = dZ W,  dW = dZ^T X                      [LLMS step 4; L27 "Trick 2"]

Readings where the pages are silent or disagree:
  * label smoothing (named in [LLMS] "Numerical Considerations" item 3 and
    [L27] "Numerical traps" without a formula): target distribution
    q_ij = (1 - eps) [j = y_i] + eps / V, so
    l_i = LSE_i - (1 - eps) z_{i,y_i} - (eps / V) sum_j z_ij and
    dL/dz_ij = (p_ij - q_ij) * g / D;
  * labels equal to ignore_index (-100) contribute no loss and no gradient
    ([LLMS] "Numerical Considerations" item 2; [CCE] chunked module);
  * mean reduction divides by D = max(N_valid, 1) ([CCE] chunked module's
    final division); sum reduction uses D = 1;
  * labels are 0-based; a label outside [0, V) that is not ignore_index is
    an error;
  * the upstream gradient g scales dX and dW.
  * z-loss ([LLMS] "Numerical Considerations" item 3 gives the term
    alpha log^2 sum_j exp(z_ij), i.e. alpha LSE_i^2 per row): it is added to
    l_i of every valid row and reduced with the same D; its derivative adds
    2 alpha LSE_i p_ij to dZ_ij;
  * reduction "none" returns the per-row losses l_i (0 on ignored rows) and
    takes a per-row upstream gradient g_i (D = 1), the form torch's
    cross_entropy(reduction="none") has;
  * the "Trick 1 only" path of [L27] ("Fused softmax+CE (keep logits, drop
    probs/dlogits)" in the logit-space memory table) is the same loss and
    dZ on logits the caller already holds: softmax_ce_on_logits below.

  * gradient filtering (CCE, [LLMS] "Apple Cut Cross-Entropy (CCE)"): see
    filtered_linear_cross_entropy for the block rule read from the page.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, invariants, finite differences and torch's fp64
cross_entropy on small shapes).  Full-size values at the five workloads
have no printed reference on the pages beyond those pins.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class OracleResult:
    loss: float
    lse: np.ndarray  # [N], NaN on ignored rows
    dX: np.ndarray  # [N, H]
    dW: np.ndarray  # [V, H]
    n_valid: int


def _as_f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def valid_rows(labels: np.ndarray, V: int, ignore_index: int = -100) -> np.ndarray:
    """Boolean mask of rows that carry a loss.  Raises on a label outside
    [0, V) that is not the ignore index (reading: an error)."""
    y = np.asarray(labels).astype(np.int64)
    keep = y != ignore_index
    bad = keep & ((y < 0) | (y >= V))
    if bad.any():
        raise ValueError(f"{int(bad.sum())} label(s) outside [0, {V}) that are not ignore_index")
    return keep


def denominator(n_valid: int, reduction: str) -> float:
    """D of the reduction: max(N_valid, 1) for "mean" ([CCE] chunked module,
    final division), 1 for "sum" and for "none" (per-row losses)."""
    if reduction == "mean":
        return float(max(n_valid, 1))
    if reduction in ("sum", "none"):
        return 1.0
    raise ValueError(f"unknown reduction {reduction!r}")


def row_scales(grad_loss, n_rows: int, D: float, reduction: str) -> np.ndarray:
    """Per-row factor of dZ: g / D for "mean" and "sum" (g a scalar), g_i
    for "none" (g a scalar broadcast or an array over the rows)."""
    g = np.asarray(grad_loss, dtype=np.float64)
    if reduction != "none" and g.ndim != 0:
        raise ValueError("grad_loss is a scalar unless reduction is 'none'")
    return np.broadcast_to(g / D, (n_rows,)).astype(np.float64)


def logits(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = X W^T ([LLMS] "The Vocabulary Memory Wall", first equation)."""
    return X @ W.T


def log_sum_exp(Z: np.ndarray) -> np.ndarray:
    """Row-wise LSE by the two-pass max-subtracted form ([LLMS] step 2;
    [CCE] "Numerical Stability": pass 1 the max, pass 2 the exponentials)."""
    m = Z.max(axis=1)
    d = np.exp(Z - m[:, None]).sum(axis=1)
    return m + np.log(d)


def token_losses(Z: np.ndarray, lse: np.ndarray, y: np.ndarray, eps: float,
                 z_loss: float = 0.0) -> np.ndarray:
    """l_i = LSE_i - (1-eps) z_{i,y_i} - (eps/V) sum_j z_ij + alpha LSE_i^2:
    the cross-entropy between the smoothed target q and softmax(z_i), plus
    the z-loss term ([LLMS] "Numerical Considerations" item 3).  For
    eps = alpha = 0 this is [LLMS] step 2's l_i = -z_{i,y_i} + m_i + log d_i."""
    V = Z.shape[1]
    z_y = Z[np.arange(Z.shape[0]), y]
    out = lse - (1.0 - eps) * z_y
    if eps != 0.0:
        out = out - (eps / V) * Z.sum(axis=1)
    if z_loss != 0.0:
        out = out + z_loss * lse * lse
    return out


def dlogits(Z: np.ndarray, lse: np.ndarray, y: np.ndarray, eps: float, scale,
            z_loss: float = 0.0) -> np.ndarray:
    """dZ_ij = (p_ij (1 + 2 alpha LSE_i) - q_ij) * scale_i with
    p_ij = exp(z_ij - LSE_i) and q_ij = (1-eps)[j = y_i] + eps/V ([LLMS]
    step 3; [L27] "The gradient that makes fusion trivial": softmax minus one
    at the true class, over N).  The z-loss factor is d(alpha LSE_i^2)/dz_ij
    = 2 alpha LSE_i p_ij.  `scale` is a scalar or one factor per row."""
    V = Z.shape[1]
    P = np.exp(Z - lse[:, None])
    if z_loss != 0.0:
        P = P * (1.0 + 2.0 * z_loss * lse)[:, None]
    P[np.arange(Z.shape[0]), y] -= 1.0 - eps
    if eps != 0.0:
        P -= eps / V
    sc = np.asarray(scale, dtype=np.float64)
    return P * (sc[:, None] if sc.ndim else sc)


def linear_cross_entropy(X, W, labels, ignore_index: int = -100, label_smoothing: float = 0.0,
                         reduction: str = "mean", grad_loss=1.0, row_block: int = 256,
                         z_loss: float = 0.0, progress=None) -> OracleResult:
    """Loss, LSE and gradients of the linear cross-entropy, fp64.

    Per block of valid rows: Z = X_b W^T, LSE, losses, dZ, then
    dX_b = dZ W and dW += dZ^T X_b ([LLMS] step 4; [L27] "Trick 2": the two
    products of the matmul backward).  Ignored rows have zero loss and zero
    gradient and an undefined (NaN) LSE.  For reduction "none" the loss is
    the array of per-row losses and grad_loss may be one value per row.
    progress: optional callable, given (valid rows done, valid rows) after
    each block (reporting only)."""
    X = _as_f64(X)
    W = _as_f64(W)
    y = np.asarray(labels).astype(np.int64)
    N, H = X.shape
    V, H2 = W.shape
    if H != H2 or y.shape != (N,):
        raise ValueError("shape mismatch")
    eps = float(label_smoothing)
    keep = valid_rows(y, V, ignore_index)
    n_valid = int(keep.sum())
    D = denominator(n_valid, reduction)
    scale = row_scales(grad_loss, N, D, reduction)

    lse = np.full(N, np.nan)
    dX = np.zeros((N, H))
    dW = np.zeros((V, H))
    per_row = np.zeros(N)
    total = 0.0
    rows = np.nonzero(keep)[0]
    for s in range(0, rows.size, max(1, int(row_block))):
        idx = rows[s:s + row_block]
        Xb = X[idx]
        Z = logits(Xb, W)
        lse_b = log_sum_exp(Z)
        terms = token_losses(Z, lse_b, y[idx], eps, z_loss)
        per_row[idx] = terms
        total += float(terms.sum())
        dZ = dlogits(Z, lse_b, y[idx], eps, scale[idx], z_loss)
        dX[idx] = dZ @ W
        dW += dZ.T @ Xb
        lse[idx] = lse_b
        if progress is not None:
            progress(s + idx.size, rows.size)
    loss = per_row if reduction == "none" else total / D
    return OracleResult(loss, lse, dX, dW, n_valid)


@dataclasses.dataclass
class FilteredResult:
    result: OracleResult  # loss and LSE exact; dX and dW from the filtered dZ
    keep: np.ndarray  # [ceil(N/tile), ceil(V/tile)] bool: tile kept
    dZ: np.ndarray  # [N, V] the filtered dZ


def filtered_linear_cross_entropy(X, W, labels, ignore_index: int = -100,
                                  label_smoothing: float = 0.0, reduction: str = "mean",
                                  grad_loss=1.0, z_loss: float = 0.0, tile: int = 256,
                                  threshold: float = 2.0 ** -12) -> FilteredResult:
    """Gradient filtering of Cut Cross-Entropy ([LLMS] "Apple Cut
    Cross-Entropy (CCE)": non-target softmax values below 2^-12 are
    negligible in bf16, and the backward skips the blocks they fill).

    Reading (the pages name neither a block shape nor what happens to the
    target term): dZ is cut into tile x tile blocks of (tokens, vocabulary)
    at multiples of `tile`; a block is dropped, i.e. treated as zero in
    dX = dZ W and dW = dZ^T X, when every softmax value p_ij of its valid
    rows is below `threshold` and none of its valid rows has its label in
    the block's columns (the target term is never dropped).  Loss and LSE
    are those of linear_cross_entropy.  Materialises N x V: small shapes."""
    full = linear_cross_entropy(X, W, labels, ignore_index, label_smoothing, reduction,
                                grad_loss, z_loss=z_loss)
    X = _as_f64(X)
    W = _as_f64(W)
    y = np.asarray(labels).astype(np.int64)
    N, V = X.shape[0], W.shape[0]
    keep_rows = valid_rows(y, V, ignore_index)
    D = denominator(int(keep_rows.sum()), reduction)
    scale = row_scales(grad_loss, N, D, reduction)
    P = np.zeros((N, V))
    dZ = np.zeros((N, V))
    idx = np.nonzero(keep_rows)[0]
    if idx.size:
        Z = logits(X[idx], W)
        lse = full.lse[idx]
        P[idx] = np.exp(Z - lse[:, None])
        dZ[idx] = dlogits(Z, lse, y[idx], label_smoothing, scale[idx], z_loss)
    nt, nv = -(-N // tile), -(-V // tile)
    keep = np.zeros((nt, nv), dtype=bool)
    for I in range(nt):
        r = slice(I * tile, min(N, (I + 1) * tile))
        yl = y[r][keep_rows[r]]
        for J in range(nv):
            c0, c1 = J * tile, min(V, (J + 1) * tile)
            has_label = bool(((yl >= c0) & (yl < c1)).any())
            big = bool((P[r, c0:c1] >= threshold).any())
            keep[I, J] = has_label or big
            if not keep[I, J]:
                dZ[r, c0:c1] = 0.0
    res = OracleResult(full.loss, full.lse, dZ @ W, dZ.T @ X, full.n_valid)
    return FilteredResult(res, keep, dZ)


def forward(X, W, labels, ignore_index=-100, label_smoothing=0.0, reduction="mean", row_block=256,
            z_loss=0.0):
    """Loss (per-row losses for "none") and per-row LSE only."""
    X = _as_f64(X)
    W = _as_f64(W)
    y = np.asarray(labels).astype(np.int64)
    keep = valid_rows(y, W.shape[0], ignore_index)
    n_valid = int(keep.sum())
    D = denominator(n_valid, reduction)
    lse = np.full(X.shape[0], np.nan)
    per_row = np.zeros(X.shape[0])
    rows = np.nonzero(keep)[0]
    for s in range(0, rows.size, max(1, int(row_block))):
        idx = rows[s:s + row_block]
        Z = logits(X[idx], W)
        lse_b = log_sum_exp(Z)
        per_row[idx] = token_losses(Z, lse_b, y[idx], label_smoothing, z_loss)
        lse[idx] = lse_b
    loss = per_row if reduction == "none" else float(per_row.sum()) / D
    return loss, lse, n_valid


def dX_rows(X, W, labels, row_idx, ignore_index=-100, label_smoothing=0.0, reduction="mean",
            grad_loss=1.0, z_loss=0.0):
    """Selected rows of dX.  Row-local except for D, which needs only the
    labels.  Returns (dX[row_idx], lse[row_idx], loss terms l_i)."""
    W = _as_f64(W)
    y = np.asarray(labels).astype(np.int64)
    N = y.shape[0]
    keep = valid_rows(y, W.shape[0], ignore_index)
    D = denominator(int(keep.sum()), reduction)
    scale = row_scales(grad_loss, N, D, reduction)
    idx = np.asarray(row_idx, dtype=np.int64)
    out = np.zeros((idx.size, W.shape[1]))
    lse = np.full(idx.size, np.nan)
    terms = np.zeros(idx.size)
    sel = keep[idx]
    if sel.any():
        Xs = _as_f64(np.asarray(X)[idx[sel]])
        Z = logits(Xs, W)
        lse_s = log_sum_exp(Z)
        dZ = dlogits(Z, lse_s, y[idx[sel]], label_smoothing, scale[idx[sel]], z_loss)
        out[sel] = dZ @ W
        lse[sel] = lse_s
        terms[sel] = token_losses(Z, lse_s, y[idx[sel]], label_smoothing, z_loss)
    return out, lse, terms


def dW_rows(X, W, labels, lse, vocab_idx, ignore_index=-100, label_smoothing=0.0,
            reduction="mean", grad_loss=1.0, z_loss=0.0):
    """Selected rows of dW: dW[v] = sum_i dZ_iv X_i over valid rows i.

    Needs the oracle's LSE of every valid row (``lse`` from :func:`forward`)."""
    X = _as_f64(X)
    W = _as_f64(W)
    y = np.asarray(labels).astype(np.int64)
    N, V = y.shape[0], W.shape[0]
    keep = valid_rows(y, V, ignore_index)
    D = denominator(int(keep.sum()), reduction)
    scale = row_scales(grad_loss, N, D, reduction)[keep]
    eps = float(label_smoothing)
    vidx = np.asarray(vocab_idx, dtype=np.int64)
    Xv = X[keep]
    yv = y[keep]
    lv = np.asarray(lse, dtype=np.float64)[keep]
    Zc = Xv @ W[vidx].T  # [N_valid, len(vidx)]: the selected logit columns
    P = np.exp(Zc - lv[:, None])
    if z_loss != 0.0:
        P = P * (1.0 + 2.0 * z_loss * lv)[:, None]
    P -= (1.0 - eps) * (yv[:, None] == vidx[None, :])
    if eps != 0.0:
        P -= eps / V
    return (P * scale[:, None]).T @ Xv


def softmax_ce_on_logits(Z, labels, ignore_index: int = -100, label_smoothing: float = 0.0,
                         reduction: str = "mean", grad_loss=1.0, z_loss: float = 0.0):
    """The same loss and dZ = dL/dZ on logits the caller holds ([L27]
    "Trick 1": probs and dlogits reuse the logits buffer).  Returns
    (loss, lse, dZ); loss is per row for "none"; ignored rows have zero dZ
    and NaN LSE."""
    Z = _as_f64(Z)
    y = np.asarray(labels).astype(np.int64)
    N, V = Z.shape
    keep = valid_rows(y, V, ignore_index)
    D = denominator(int(keep.sum()), reduction)
    scale = row_scales(grad_loss, N, D, reduction)
    lse = np.full(N, np.nan)
    dZ = np.zeros((N, V))
    per_row = np.zeros(N)
    idx = np.nonzero(keep)[0]
    if idx.size:
        Zv = Z[idx]
        lse_v = log_sum_exp(Zv)
        lse[idx] = lse_v
        per_row[idx] = token_losses(Zv, lse_v, y[idx], label_smoothing, z_loss)
        dZ[idx] = dlogits(Zv, lse_v, y[idx], label_smoothing, scale[idx], z_loss)
    loss = per_row if reduction == "none" else float(per_row.sum()) / D
    return loss, lse, dZ
