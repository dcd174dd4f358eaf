"""Logit-space memory accounting (host arithmetic, no GPU).

The pages count logit-space device memory under three conventions:
  * one N x V tensor of the storage dtype ("Chunked and Fused Cross-Entropy",
    llms.blog, "The Vocabulary Memory Wall"; aifetchly "The Logit Memory
    Wall", fp32 logits);
  * logits plus their gradient, 2 x N x V (llms.blog, "VRAM Footprint Across
    Model Families" table, whose fused column is two 512-row blocks);
  * logits, probabilities and their gradient, 3 x N x V ("Fused
    cross-entropy -- the memory kernel", "Worked number" table).
The fused path of this library keeps exactly one logit-space buffer, the
backward's dZ block (fce_plan's scratch_bytes).
"""
from __future__ import annotations

GB = 1e9


def logit_space_bytes(rows: int, V: int, dtype_bytes: int = 2, copies: int = 1) -> int:
    """Bytes of ``copies`` tensors of ``rows`` x V elements."""
    return int(copies) * int(rows) * int(V) * int(dtype_bytes)


def report(N: int, V: int, dtype_bytes: int, scratch_bytes: int) -> dict:
    """Naive figures under the pages' conventions next to the fused scratch."""
    return {
        "naive_1x_bytes": logit_space_bytes(N, V, dtype_bytes, 1),
        "naive_2x_bytes": logit_space_bytes(N, V, dtype_bytes, 2),
        "naive_3x_bytes": logit_space_bytes(N, V, dtype_bytes, 3),
        "fused_scratch_bytes": int(scratch_bytes),
    }
