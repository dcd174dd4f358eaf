"""Write the oracle's expected values for the full-size workloads 2-5.

Calls only the seeded input generator (``workloads``) and the fp64 oracle
(``oracle``).  For each workload it stores, in tests/golden/oracle_config<k>.npz:
  digest        sha256 of the drawn inputs (guards against generator drift)
  loss, n_valid the oracle's mean loss and valid-token count
  lse           LSE of every row (float32; NaN on ignored rows)
  dx_idx, dx    sampled rows of dX (float32)
  dw_idx, dw    sampled rows of dW (float32)
The sampled rows include ignored rows, the first and last row, the most
frequent label and the last vocabulary entry.

Usage: python tests/golden/make_oracle_goldens.py [k ...]
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle.fce_oracle as orc  # noqa: E402
import workloads as wk  # noqa: E402

OUT = os.path.dirname(os.path.abspath(__file__))


def sample_rows(inp):
    N, V = inp.workload.N, inp.workload.V
    g = np.random.default_rng(inp.workload.seed + 7)
    y = inp.labels
    ign = np.nonzero(y == wk.IGNORE_INDEX)[0]
    dx = [0, 1, N // 2, N - 1] + list(ign[:2]) + list(g.choice(N, 2, replace=False))
    valid = y[y != wk.IGNORE_INDEX]
    vals, counts = np.unique(valid, return_counts=True)
    head = int(vals[np.argmax(counts)])
    dw = [0, V - 1, int(valid[0]), head] + list(g.choice(V, 2, replace=False))
    return np.array(sorted(set(int(i) for i in dx))), np.array(sorted(set(int(v) for v in dw)))


def make(k):
    wl = wk.WORKLOADS[k]
    t0 = time.time()
    inp = wk.draw(wl)
    eps = wl.label_smoothing
    loss, lse, n_valid = orc.forward(inp.X, inp.W, inp.labels, wk.IGNORE_INDEX, eps, "mean",
                                     row_block=256)
    dx_idx, dw_idx = sample_rows(inp)
    dx, _, _ = orc.dX_rows(inp.X, inp.W, inp.labels, dx_idx, wk.IGNORE_INDEX, eps, "mean")
    dw = orc.dW_rows(inp.X, inp.W, inp.labels, lse, dw_idx, wk.IGNORE_INDEX, eps, "mean")
    path = os.path.join(OUT, f"oracle_config{k}.npz")
    np.savez_compressed(path, digest=np.array(inp.digest()), loss=np.float64(loss),
                        n_valid=np.int64(n_valid), lse=lse.astype(np.float32),
                        dx_idx=dx_idx, dx=dx.astype(np.float32), dw_idx=dw_idx,
                        dw=dw.astype(np.float32))
    print(f"config {k} ({wl.name}): loss {loss:.8f} n_valid {n_valid} "
          f"[{time.time() - t0:.1f}s] -> {path}", flush=True)


if __name__ == "__main__":
    ks = [int(a) for a in sys.argv[1:]] or [2, 3, 4, 5]
    for k in ks:
        make(k)
