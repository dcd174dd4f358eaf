"""Errors measured by the GPU parity tests, for the end-of-run summary.

Tests call ``record`` with the quantities they assert on (relative error of
the loss, relative L2 error of the LSE, dX and dW against the fp64 oracle)
and the bound each is held to; tests/conftest.py prints every record after
the run, so the margins show in the log of a passing run too.
"""
RECORDS = []


def record(name: str, bound_loss: float, bound_grad: float, **errors) -> None:
    """One parity check: ``errors`` maps a quantity (loss, lse, dX, dW, dZ,
    ...) to its measured error."""
    RECORDS.append((name, bound_loss, bound_grad, dict(errors)))


def summary_lines():
    out = []
    for name, bl, bg, errs in RECORDS:
        parts = " ".join(f"{k} {v:.2e}" for k, v in errs.items())
        out.append(f"{name}: {parts} (bounds: loss/lse {bl:.0e}, grads {bg:.0e})")
    return out
