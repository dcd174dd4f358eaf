"""Seeded synthetic inputs for fused linear cross-entropy.

This module only draws inputs: hidden states X[N,H], unembedding weights
W[V,H] and int32 labels[N].  It holds none of the loss arithmetic, so the
CPU oracle and the HIP path can both be fed from it without sharing code.

The five named workloads mirror the shapes the pages discuss (a Llama-2-like
32k vocabulary, the Llama-3-8B shape of the "Worked number" table on the
"Fused cross-entropy -- the memory kernel" page, and the Qwen2.5 / Gemma-2
vocabularies of the "VRAM Footprint Across Model Families" table on the
llms.blog page).  Only the shapes are used; values are random.

Recipe (every array is a pure function of the workload's seed):
  * numpy ``SeedSequence(20261200 + k)`` for workload k, spawned in fixed
    order into five streams: X, W, labels, vocabulary permutation, ignore
    positions.
  * X ~ N(0, 1) and W ~ N(0, sigma^2), drawn in float32 in fixed slabs of
    rows (each slab has its own spawned child seed, so the result does not
    depend on how many threads fill it), then rounded to bfloat16 with
    round-to-nearest-even (the fp32 workload keeps float32).
  * Labels: uniform on [0, V), or a truncated Zipf law P(rank k) ~ k^-s over
    ranks 1..V sampled by inverse CDF and mapped through a random
    permutation of the vocabulary.
  * Exactly round(p * N) positions, drawn without replacement, are set to
    ``ignore_index`` (-100).
  * ``draw_logits`` (inputs of the loss on given logits): the same labels,
    and logits Z[N,V] ~ N(0, (sigma sqrt(H))^2) -- the scale X W^T has for
    this workload -- from a sixth spawned stream, in slabs of 256 rows,
    rounded to bfloat16 like X and W.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

IGNORE_INDEX = -100
SEED_BASE = 20261200
_SLAB_ROWS = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value distribution of one synthetic workload."""

    name: str
    N: int
    H: int
    V: int
    dtype: str  # "fp32" or "bf16": storage and arithmetic type of X and W
    w_sigma: float
    label_dist: str  # "uniform" or "zipf"
    zipf_s: float
    ignore_frac: float
    label_smoothing: float
    seed: int

    @property
    def n_ignored(self) -> int:
        return int(round(self.ignore_frac * self.N))


WORKLOADS = {
    1: Workload("tiny-fp32", 256, 128, 4096, "fp32", 0.05, "uniform", 0.0, 0.0, 0.0, SEED_BASE + 1),
    2: Workload("llama2-32k", 4096, 2048, 32000, "bf16", 0.02, "uniform", 0.0, 0.05, 0.0, SEED_BASE + 2),
    3: Workload("llama3-8b", 8192, 4096, 128256, "bf16", 0.02, "zipf", 1.1, 0.02, 0.0, SEED_BASE + 3),
    4: Workload("qwen2.5-7b-ls", 16384, 3584, 152064, "bf16", 0.02, "zipf", 1.1, 0.03, 0.1, SEED_BASE + 4),
    5: Workload("gemma2-2b", 32768, 2304, 256000, "bf16", 0.03, "zipf", 1.2, 0.01, 0.0, SEED_BASE + 5),
}


def custom(N, H, V, dtype="bf16", w_sigma=0.02, label_dist="uniform", zipf_s=1.1,
           ignore_frac=0.0, label_smoothing=0.0, seed=1, name="custom") -> Workload:
    return Workload(name, N, H, V, dtype, w_sigma, label_dist, zipf_s, ignore_frac,
                    label_smoothing, seed)


@dataclasses.dataclass
class Inputs:
    """One drawn instance.  ``X``/``W`` hold the exact stored values as
    float32 (bf16 values are exactly representable in float32); for bf16
    workloads ``X_bits``/``W_bits`` hold the raw bfloat16 bit patterns."""

    workload: Workload
    X: np.ndarray
    W: np.ndarray
    labels: np.ndarray
    X_bits: np.ndarray | None
    W_bits: np.ndarray | None

    @property
    def ignore_index(self) -> int:
        return IGNORE_INDEX

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.X, self.W, self.labels):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.
    Inputs here are finite draws, so NaN/Inf handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_matrix(ss: np.random.SeedSequence, rows: int, cols: int, sigma: float) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    n_slabs = max(1, -(-rows // _SLAB_ROWS))
    children = ss.spawn(n_slabs)

    def fill(i):
        r0 = i * _SLAB_ROWS
        r1 = min(rows, r0 + _SLAB_ROWS)
        if r1 <= r0:
            return
        g = np.random.Generator(np.random.PCG64(children[i]))
        view = out[r0:r1]
        g.standard_normal(out=view, dtype=np.float32)
        if sigma != 1.0:
            np.multiply(view, np.float32(sigma), out=view)

    if n_slabs == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_slabs)))
    return out


def _zipf_ranks(g: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """Truncated Zipf on ranks 1..V by inverse CDF; returns 0-based ranks."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = g.random(n)
    r = np.searchsorted(cdf, u, side="right")
    return np.minimum(r, V - 1)


def _labels(wl: Workload, s_lab, s_perm, s_ign) -> np.ndarray:
    g_lab = np.random.Generator(np.random.PCG64(s_lab))
    if wl.label_dist == "uniform":
        labels = g_lab.integers(0, wl.V, size=wl.N, dtype=np.int64)
    elif wl.label_dist == "zipf":
        ranks = _zipf_ranks(g_lab, wl.N, wl.V, wl.zipf_s)
        perm = np.random.Generator(np.random.PCG64(s_perm)).permutation(wl.V)
        labels = perm[ranks]
    else:
        raise ValueError(f"unknown label distribution {wl.label_dist!r}")
    labels = labels.astype(np.int32)

    k = wl.n_ignored
    if k > 0:
        pos = np.random.Generator(np.random.PCG64(s_ign)).choice(wl.N, size=k, replace=False)
        labels[pos] = IGNORE_INDEX
    return labels


def draw(wl: Workload) -> Inputs:
    """Draw the inputs of a workload (deterministic in ``wl.seed``)."""
    s_x, s_w, s_lab, s_perm, s_ign = np.random.SeedSequence(wl.seed).spawn(5)
    X = _normal_matrix(s_x, wl.N, wl.H, 1.0)
    W = _normal_matrix(s_w, wl.V, wl.H, wl.w_sigma)
    labels = _labels(wl, s_lab, s_perm, s_ign)

    X_bits = W_bits = None
    if wl.dtype == "bf16":
        X_bits = round_to_bf16_bits(X)
        W_bits = round_to_bf16_bits(W)
        X = bf16_bits_to_f32(X_bits)
        W = bf16_bits_to_f32(W_bits)
    elif wl.dtype != "fp32":
        raise ValueError(f"unknown dtype {wl.dtype!r}")
    return Inputs(wl, X, W, labels, X_bits, W_bits)


@dataclasses.dataclass
class LogitInputs:
    """Inputs of the loss on given logits: Z holds the stored values as
    float32; Z_bits the bfloat16 bit patterns for bf16 workloads."""

    workload: Workload
    Z: np.ndarray
    labels: np.ndarray
    Z_bits: np.ndarray | None

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.Z, self.labels):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def draw_logits(wl: Workload) -> LogitInputs:
    """Logits and labels for the loss on given logits (deterministic in
    ``wl.seed``; the labels equal those of :func:`draw`)."""
    s_x, s_w, s_lab, s_perm, s_ign, s_z = np.random.SeedSequence(wl.seed).spawn(6)
    labels = _labels(wl, s_lab, s_perm, s_ign)
    sigma = float(wl.w_sigma) * float(np.sqrt(wl.H))
    Z = np.empty((wl.N, wl.V), dtype=np.float32)
    rows = 256
    children = s_z.spawn(max(1, -(-wl.N // rows)))

    def fill(i):
        r0, r1 = i * rows, min(wl.N, (i + 1) * rows)
        g = np.random.Generator(np.random.PCG64(children[i]))
        view = Z[r0:r1]
        g.standard_normal(out=view, dtype=np.float32)
        np.multiply(view, np.float32(sigma), out=view)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(children))))
    Z_bits = None
    if wl.dtype == "bf16":
        Z_bits = np.empty(Z.shape, dtype=np.uint16)

        def conv(i):
            r0, r1 = i * rows, min(wl.N, (i + 1) * rows)
            Z_bits[r0:r1] = round_to_bf16_bits(Z[r0:r1])
            Z[r0:r1] = bf16_bits_to_f32(Z_bits[r0:r1])

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(len(children))))
    return LogitInputs(wl, Z, labels, Z_bits)


def logits_to_torch(inp: LogitInputs, device="cuda"):
    """Z as a torch tensor of the workload dtype and int32 labels, on ``device``."""
    import torch

    if inp.workload.dtype == "bf16":
        Z = torch.from_numpy(inp.Z_bits.view(np.int16)).view(torch.bfloat16)
    else:
        Z = torch.from_numpy(inp.Z)
    return Z.to(device), torch.from_numpy(inp.labels).to(device)


def to_torch(inp: Inputs, device="cuda"):
    """X, W as torch tensors of the workload dtype and int32 labels, on ``device``."""
    import torch

    if inp.workload.dtype == "bf16":
        X = torch.from_numpy(inp.X_bits.view(np.int16)).view(torch.bfloat16)
        W = torch.from_numpy(inp.W_bits.view(np.int16)).view(torch.bfloat16)
    else:
        X = torch.from_numpy(inp.X)
        W = torch.from_numpy(inp.W)
    y = torch.from_numpy(inp.labels)
    return X.to(device), W.to(device), y.to(device)
