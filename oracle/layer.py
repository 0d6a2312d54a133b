"""A token through whole decoder layers, in float64 -- test infrastructure.

"src/families/qwen4/mod.rs", module doc, "The decoder layer, as pseudocode": at entry the
token's hidden vector is replicated over the C streams (not padded); each layer runs

    mixed, raw, inject_w = attn_hc(hidden);  out = attention_sublayer(mixed)
    hidden = raw + (out[None, :] * inject_w[:, None]).flatten()
    mixed, raw, inject_w = mlp_hc(hidden);   out = moe(mixed)
    hidden = raw + (out[None, :] * inject_w[:, None]).flatten()

and at exit the hyper_connection_mixer (the same read with no inject projection) collapses the
C*H residual to H. The attention sublayer is outside the hot path this package builds; it is
replaced here by a plain INT4-affine H x H linear map ("the stand-in").

Every tensor the composition stores between steps is rounded to the dtype it is stored in:
mixed, each sublayer output and the residual after each inject to fp16 (the widths and fp16
storage of these tensors are those of the hyper-connection and MoE workloads), and the inject
weights to fp32. Each step is the pinned oracle function of its own module (hc_read,
hc_inject, dequant_gemv, moe_decode).

Parity: pinned through its steps; tests/test_oracle_layer.py adds the composition's own pins
(identity stand-in and zero experts reduce a layer to hand-computed injects; replicated entry;
the residual, not the normed stream, carries the inject).
"""
from __future__ import annotations

import numpy as np

from .gemv import dequant_gemv
from .hc import hc_inject, hc_read
from .moe import moe_decode


def _f16(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


def _f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def decode_layers(x, layers, mixer, C: int, H: int, eps: float = 1e-6):
    """x fp16 [H]; layers: list of dict(attn, stub, mlp, moe) with attn/mlp = dict(gamma_bits,
    down, up, inject), stub an Int4 [H x H], moe = dict(router_bits, sgate_bits, shared,
    experts, top_k[, fp16_boundary]); mixer = dict(gamma_bits, down, up).

    Returns dict(hidden [C*H] after the last layer, mixed [H] from the mixer, ids per layer).
    """
    hidden = np.tile(np.asarray(x, dtype=np.float64), C)          # entry replication
    ids = []
    for L in layers:
        a = L["attn"]
        r = hc_read(hidden, a["gamma_bits"], a["down"], a["up"], a["inject"], C, H, eps)
        out = _f16(dequant_gemv(L["stub"].q, L["stub"].s_bits, L["stub"].b_bits, _f16(r["mixed"])))
        hidden = _f16(hc_inject(hidden, out, _f32(r["inject_w"]), C, H))
        m = L["mlp"]
        r = hc_read(hidden, m["gamma_bits"], m["down"], m["up"], m["inject"], C, H, eps)
        e = L["moe"]
        d = moe_decode(_f16(r["mixed"]), e["router_bits"], e["sgate_bits"], e["shared"], e["experts"], e["top_k"],
                       fp16_boundary=e.get("fp16_boundary", False))
        ids.append(d["ids"])
        hidden = _f16(hc_inject(hidden, _f16(d["out"]), _f32(r["inject_w"]), C, H))
    mixed = _f16(hc_read(hidden, mixer["gamma_bits"], mixer["down"], mixer["up"], None, C, H, eps)["mixed"])
    return {"hidden": hidden, "mixed": mixed, "ids": ids}
