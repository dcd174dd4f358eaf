"""fp64 CPU oracle for linear cross-entropy.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path."""
from .fce_oracle import (  # noqa: F401
    OracleResult,
    dlogits,
    dW_rows,
    dX_rows,
    denominator,
    forward,
    linear_cross_entropy,
    log_sum_exp,
    logits,
    token_losses,
    valid_rows,
)
