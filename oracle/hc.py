"""Hyper-connection read and inject for one token, in float64 (test infrastructure: only the
tests, the smoke check and the benchmark's CPU baseline use this package).

Defined by "src/families/qwen4/mod.rs", section "Hyper-connections" (with its decoder-layer
pseudocode and the note on the injection trap), and by "src/families/qwen4/hc.rs",
encode_hyper_connection. The residual holds C streams of width H; element (c, h) sits at
index c*H + h. Written per element, with W_d [R x C*H], W_u [C*H x R], W_i [C x C*H] the
three INT4-affine projections (the pages run them through a dtype-generic GEMV) and
gamma the stored norm weight:

  rho[c]      = sqrt( (1/H) * sum_h raw[c,h]^2 + eps )            one RMS per stream
  n[c,h]      = raw[c,h] / rho[c] * gamma[c,h]                     gamma applied as stored,
                                                                   not as 1 + gamma (hc.rs doc)
  lo[r]       = silu( (1/C) * sum_{c,h} W_d[r, c*H+h] * n[c,h] )   first of the two 1/C
  u[c,h]      = sigmoid( sum_r W_u[c*H+h, r] * lo[r] )             no 1/C on this projection
  mixed[h]    = (1/C) * sum_c u[c,h] * n[c,h]                      a mean over streams, not a sum
  iw[c]       = 2 * sigmoid( (1/C) * sum_{c',h} W_i[c, c'*H+h] * n[c',h] )   second 1/C;
                                                                   absent on the final mixer
  hidden[c,h] = raw[c,h] + out[h] * iw[c]                          the sublayer output lands on
                                                                   the un-normalized stream

with eps = 1e-6 (the qwen4 page's RMS epsilon) and silu(z) = z * sigmoid(z).

Parity: pinned (constant-input norm closed form, per-group independence, scale
invariance, zero-weight closed forms for u = 1/2 and iw = 1, selector closed forms
that fix both 1/C divisions and the mean, C=1 plain residual add, hand-worked C=2
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
    """n[c,h] = raw[c,h] / rho[c] * gamma[c,h], rho[c] = sqrt(mean_h raw[c,h]^2 + eps); flat [C*H]."""
    x = np.asarray(raw, dtype=np.float64).reshape(C, H)
    g = bf16_bits_to_f64(gamma_bits).reshape(C, H)
    rho = np.sqrt(np.sum(x * x, axis=1) / H + eps)
    return (x / rho[:, None] * g).reshape(C * H)


def _project(w, v) -> np.ndarray:
    """sum_j W[i, j] * v[j] for an INT4-affine W, in float64."""
    return dequant_gemv(w.q, w.s_bits, w.b_bits, v)


def hc_read(raw, gamma_bits, down, up, inject, C: int, H: int, eps: float = RMS_EPS):
    """One hyper-connection read. ``inject`` may be None (the final mixer).

    Returns dict(mixed [H], inject_w [C] or None, normed [C*H], lo [R], u [C*H]).
    """
    n = grouped_rmsnorm(raw, gamma_bits, C, H, eps)
    lo = _silu(_project(down, n) / C)
    u = _sigmoid(_project(up, lo))
    mixed = np.sum(u.reshape(C, H) * n.reshape(C, H), axis=0) / C
    iw = None
    if inject is not None:
        iw = 2.0 * _sigmoid(_project(inject, n) / C)
    return {"mixed": mixed, "inject_w": iw, "normed": n, "lo": lo, "u": u}


def hc_inject(raw, out, inject_w, C: int, H: int) -> np.ndarray:
    """hidden[c*H + h] = raw[c*H + h] + out[h] * iw[c], in float64; flat [C*H]."""
    r = np.asarray(raw, dtype=np.float64).reshape(C, H)
    o = np.asarray(out, dtype=np.float64)
    w = np.asarray(inject_w, dtype=np.float64)
    hidden = np.empty((C, H), dtype=np.float64)
    for c in range(C):
        hidden[c] = r[c] + o * w[c]
    return hidden.reshape(C * H)


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

