"""INT4-affine weights as the decode runtime stores them, decoded in float64.

"src/real_forward.rs", module doc, memory model: every projection binds
weights / scales / biases of an INT4-affine tensor resident in one buffer. The pages
do not print the element formula; the plainest reading of "affine" with a separate
scale and bias per group is

    W[n, k] = q[n, k] * s[n, k // 64] + b[n, k // 64]

with unsigned codes q in 0..15 and a group of 64 consecutive k. The group size and
the bf16 storage of s and b come from the workload definitions, not the pages.

Parity: pinned (closed-form code table, group-index selector test).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant(q, s_bits, b_bits, group: int = GROUP) -> np.ndarray:
    """W[n,k] = q[n,k] * s[n, k//group] + b[n, k//group], all in float64."""
    q = np.asarray(q)
    n, k = q.shape
    if k % group:
        raise ValueError(f"K={k} is not a multiple of the group size {group}")
    if q.min(initial=0) < 0 or q.max(initial=0) > 15:
        raise ValueError("INT4 codes must lie in 0..15")
    s = bf16_bits_to_f64(s_bits).reshape(n, k // group)
    b = bf16_bits_to_f64(b_bits).reshape(n, k // group)
    return q.astype(np.float64) * np.repeat(s, group, axis=1) + np.repeat(b, group, axis=1)
