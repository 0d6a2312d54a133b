"""Dequantizing GEMV / GEMM and the LM-head argmax, in float64.

"src/real_forward.rs": module doc (dequant_int4_gemv_simd against resident INT4-affine
weights) and field batched_gemv_prefill (the M-row GEMM computes exactly the same
outputs as M independent GEMVs). So

    Y[m, n] = sum_k W[n, k] * X[m, k]

for every row m of the activations, with W from oracle.int4.dequant. The LM head of
"src/families/qwen4/mod.rs" (decoder-layer pseudocode, exit: logits = lm_head(hidden))
is the same product over the vocabulary; its logits are fp32, so the argmax is taken
on the fp32-rounded logits and the lowest index wins a tie.

Parity: pinned (unit-vector columns, exact rational brute force, constant-code closed
form, planted maxima and ties).
"""
from __future__ import annotations

import numpy as np

from .int4 import dequant


def dequant_gemv(q, s_bits, b_bits, x, row_chunk: int = 4096) -> np.ndarray:
    """Y[m, n] = sum_k W[n,k] X[m,k] in float64. x is [K] or [M, K]; returns [N] or [M, N].

    Rows of W are dequantized ``row_chunk`` at a time to bound memory; each output is
    still one float64 dot product (the BLAS routine picks its own summation order).
    """
    x64 = np.asarray(x, dtype=np.float64)
    squeeze = x64.ndim == 1
    X = x64[None, :] if squeeze else x64
    q = np.asarray(q)
    n = q.shape[0]
    s_bits = np.asarray(s_bits)
    b_bits = np.asarray(b_bits)
    Y = np.empty((X.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        W = dequant(q[r0:r1], s_bits[r0:r1], b_bits[r0:r1])
        Y[:, r0:r1] = X @ W.T
    return Y[0] if squeeze else Y


def argmax_lowest(logits) -> np.ndarray:
    """Per-row index of the maximum of the fp32-rounded logits; lowest index on ties."""
    L = np.asarray(logits, dtype=np.float64)
    L32 = L.astype(np.float32)
    if L32.ndim == 1:
        return np.int64(np.argmax(L32))   # numpy returns the first occurrence of the max
    return np.argmax(L32, axis=1).astype(np.int64)
