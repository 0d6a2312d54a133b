"""Hyper-connection read and inject for one token, in float64.

"src/families/qwen4/mod.rs", section "Hyper-connections", and "src/families/qwen4/hc.rs",
encode_hyper_connection. With C streams of width H (residual C*H wide), in the pages'
order:

    normed  = grouped RMS norm of raw, one group per stream, scaled directly by hc_norm
    lo      = silu(down(normed) / C)                      C*H -> R
    u       = sigmoid(up(lo))                             R -> C*H, no 1/C here
    mixed   = mean over the C streams of u * normed       -> H
    inject  = 2 * sigmoid(block_inject(normed) / C)       C*H -> C  (absent on the final mixer)

and the inject of the decoder-layer pseudocode (same page, "The decoder layer, as
pseudocode", and "THE INJECTION TRAP"): the sublayer output is added to the
UN-normalized raw stream, scaled per stream,

    hidden[c*H + h] = raw[c*H + h] + out[h] * inject[c].

RMS norm: x / sqrt(mean(x^2) + eps) * weight with eps = RMS_EPS = 1e-6 (constant on the
qwen4 page); the weight multiplies directly (hc.rs doc: the stored GGUF scale is
applied as is, not as 1 + w). The three projections are INT4-affine GEMVs here (the
pages dispatch them through a dtype-generic GEMV).

Parity: pinned (constant-input norm closed form, per-group independence, scale
invariance, zero-weight closed forms for u = 1/2 and inject = 1, selector closed forms
that fix both 1/C divisions and the MEAN, C=1 plain residual add, hand-worked C=2
inject fixture; mutated oracles with a third 1/C, a sum for the mean, or the inject
into the normed stream fail these pins).
"""
from __future__ import annotations

import numpy as np

from .int4 import bf16_bits_to_f64
from .gemv import dequant_gemv

RMS_EPS = 1e-6


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def grouped_rmsnorm(raw, gamma_bits, C: int, H: int, eps: float = RMS_EPS) -> np.ndarray:
    """n[c,h] = raw[c,h] / sqrt(mean_h raw[c,:]^2 + eps) * gamma[c,h]; returns flat [C*H]."""
    x = np.asarray(raw, dtype=np.float64).reshape(C, H)
    g = bf16_bits_to_f64(gamma_bits).reshape(C, H)
    rms = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return (x / rms * g).reshape(C * H)


def hc_read(raw, gamma_bits, down, up, inject, C: int, H: int, eps: float = RMS_EPS):
    """One hyper-connection call. ``inject`` may be None (the final mixer).

    Returns dict(mixed [H], inject_w [C] or None, normed, lo, u).
    """
    n = grouped_rmsnorm(raw, gamma_bits, C, H, eps)
    lo = _silu(dequant_gemv(down.q, down.s_bits, down.b_bits, n) / C)
    u = _sigmoid(dequant_gemv(up.q, up.s_bits, up.b_bits, lo))
    mixed = (u.reshape(C, H) * n.reshape(C, H)).mean(axis=0)
    iw = None
    if inject is not None:
        iw = 2.0 * _sigmoid(dequant_gemv(inject.q, inject.s_bits, inject.b_bits, n) / C)
    return {"mixed": mixed, "inject_w": iw, "normed": n, "lo": lo, "u": u}


def hc_inject(raw, out, inject_w, C: int, H: int) -> np.ndarray:
    """hidden = raw + (out[None, :] * inject_w[:, None]).flatten(), in float64; flat [C*H]."""
    r = np.asarray(raw, dtype=np.float64).reshape(C, H)
    o = np.asarray(out, dtype=np.float64).reshape(1, H)
    w = np.asarray(inject_w, dtype=np.float64).reshape(C, 1)
    return (r + o * w).reshape(C * H)


def hc_read_batched(raw_rows, gamma_bits, down, up, inject, C: int, H: int, eps: float = RMS_EPS):
    """The read for the m tokens of a chunked-prefill micro-batch: "src/families/qwen4/hc.rs",
    encode_hyper_connection, run once per token (each token's inject gate in its own row). So
    the definition is hc_read on each row. Returns dict(mixed [m, H], inject_w [m, C] or None)."""
    rows = [hc_read(r, gamma_bits, down, up, inject, C, H, eps) for r in np.asarray(raw_rows)]
    iw = None if inject is None else np.stack([r["inject_w"] for r in rows])
    return {"mixed": np.stack([r["mixed"] for r in rows]), "inject_w": iw}


def hc_inject_batched(raw_rows, out_rows, inject_w_rows, C: int, H: int) -> np.ndarray:
    """hc_inject on each row of a chunk, each with its own gate row; [m, C*H]."""
    return np.stack([hc_inject(r, o, w, C, H) for r, o, w in zip(raw_rows, out_rows, inject_w_rows)])

