"""Routed mixture-of-experts decode for one token, in float64.

Steps, in the order the pages give them:

1. Router GEMV. "src/families/qwen/state.rs", struct RealQwenState: the router output
   is an fp32 buffer of one logit per expert (router_logits_f32). The INT8 router
   kernel multiplies each x[n] by an effective per-element scale before the dot
   products (router_ones, a bf16 [hidden] buffer), so in general
   logits[e] = sum_n R[e][n] * (scale[n] * x[n]); for this family the scale is all ones
   and the logits are the plain product R @ x. R may be bf16, fp32 or INT8 codes (the
   codes' values are the weights; an INT8 router's scale lives in the per-element scale).
2. Selection. "src/families/qwen4/mod.rs", section "MoE": top-k is taken on the raw
   logits and the softmax runs over the selected set only (equivalently: softmax over
   all, top-k, renormalize -- no router bias). The logits are fp32 on the pages, so
   the selection is decided on the fp32-rounded values; ties go to the lowest expert
   index (reading: the pages are silent on ties) and the selected ids are returned in
   order of decreasing logit. The per-expert scale ("src/families/qwen/state.rs",
   per_expert_ones, the weighting of the shared top-k routine) multiplies each selected
   expert's softmax weight afterwards (reading: after the renormalization, not renormalized
   again, and never part of the selection); all ones for this family. The section's
   "top-10 renormalization" and the model check on the streamed-expert slot count give
   k <= 10.
3. Phase 1. "src/real_forward.rs", module doc: the phase-1 kernel runs each selected
   expert's gate and up projections and the gated-FFN activation, act = silu(gate)*up.
4. Phase 2: each selected expert's down projection, weighted by its softmax weight and
   reduced over the k experts.
5. Shared expert. "src/families/qwen/state.rs": the shared expert is gated by a scalar
   logit (shared_gate_logit) through a sigmoid and added to the routed sum (h1, h2).
6. Output rounding. Default: one rounding of routed + shared to fp16 at the end.
   Optional "fp16 boundary" reading of "src/families/qwen4/mod.rs", section "MoE"
   (the routed sum is cast to the model dtype before the gated shared expert is added):
   routed and gated-shared are each rounded to fp16 before the add.

Parity: pinned (top-k against exhaustive subset search, k up to 10; softmax closed form for
two experts; the pages' softmax-order identity; weights sum to one; identical-experts
invariant; selector-weight closed forms for gate/up/down and the shared gate; the router
scales: a one-hot per-element scale gives one column of R times x[n], a power-of-two scale
multiplies the logits exactly, INT8 one-hot rows incl. code -128 give signed x values, the
per-expert scale of a top-1 route is its weight and never changes the selection; the fp16
boundary by hand-built layers whose routed sum is 1 + 2^-12 and whose gated shared half is
1/2 + 2^-13, values that fp16 rounds to 1 and 1/2).
"""
from __future__ import annotations

import math

import numpy as np

from .int4 import bf16_bits_to_f64
from .gemv import dequant_gemv


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def router_logits(router, x, router_is_bf16_bits: bool = True, elem_scale_bits=None) -> np.ndarray:
    """l[e] = sum_n R[e,n] (s[n] x[n]) in float64 (R given as bf16 bits, or as values: fp32
    weights or INT8 codes; s the bf16 per-element scale, ones when None)."""
    R = bf16_bits_to_f64(router) if router_is_bf16_bits else np.asarray(router, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    if elem_scale_bits is not None:
        x = bf16_bits_to_f64(elem_scale_bits) * x
    return R @ x


def select_topk(logits, k: int) -> np.ndarray:
    """Indices of the k largest fp32-rounded logits, largest first, lowest index on ties."""
    l32 = np.asarray(logits, dtype=np.float64).astype(np.float32).astype(np.float64)
    if not 1 <= k <= l32.shape[0]:
        raise ValueError(f"top_k={k} outside 1..{l32.shape[0]}")
    order = sorted(range(l32.shape[0]), key=lambda e: (-l32[e], e))
    return np.asarray(order[:k], dtype=np.int64)


def softmax_selected(logits, ids) -> np.ndarray:
    """w_j = exp(l[ids_j]) / sum_i exp(l[ids_i]) over the selected set (fp32-rounded logits)."""
    l32 = np.asarray(logits, dtype=np.float64).astype(np.float32).astype(np.float64)
    sel = l32[np.asarray(ids)]
    e = np.exp(sel - sel.max())
    return e / e.sum()


def expert_act(expert, x) -> np.ndarray:
    """Phase 1 for one expert: silu(G x) * (U x), G and U INT4-affine [inter x hidden]."""
    g = dequant_gemv(expert["gate"].q, expert["gate"].s_bits, expert["gate"].b_bits, x)
    u = dequant_gemv(expert["up"].q, expert["up"].s_bits, expert["up"].b_bits, x)
    return silu(g) * u


def expert_down(expert, act) -> np.ndarray:
    """Phase 2 for one expert: D act, D INT4-affine [hidden x inter]."""
    d = expert["down"]
    return dequant_gemv(d.q, d.s_bits, d.b_bits, act)


def combine(routed, shared_gated, fp16_boundary: bool = False) -> np.ndarray:
    """The layer output from its two halves. Default: routed + shared_gated, unrounded (the
    caller rounds once to fp16). fp16 boundary ("src/families/qwen4/mod.rs", section "MoE": the
    routed expert sum is cast to the model dtype before the gated shared expert is added): each
    half is rounded to fp16 (round to nearest even) first, then they are added."""
    routed = np.asarray(routed, dtype=np.float64)
    shared_gated = np.asarray(shared_gated, dtype=np.float64)
    if fp16_boundary:
        return routed.astype(np.float16).astype(np.float64) + shared_gated.astype(np.float16).astype(np.float64)
    return routed + shared_gated


def moe_decode(x, router_bits, sgate_bits, shared, experts, top_k: int,
               fp16_boundary: bool = False, router_is_bf16_bits: bool = True, elem_scale_bits=None,
               expert_scale=None):
    """Full MoE decode for one token.

    ``experts`` is indexable by expert id (a list, or a dict holding at least the
    selected ids). elem_scale_bits: bf16 [hidden] per-element router scale, expert_scale:
    fp32 [E] per-expert weight scale (None: ones; the shared gate row takes neither).
    Returns dict(out, ids, weights, logits, routed, shared_gated, gate).
    """
    x = np.asarray(x, dtype=np.float64)
    logits = router_logits(router_bits, x, router_is_bf16_bits, elem_scale_bits)
    ids = select_topk(logits, top_k)
    w = softmax_selected(logits, ids)
    if expert_scale is not None:
        w = w * np.asarray(expert_scale, dtype=np.float64)[ids]
    routed = np.zeros(shared["down"].q.shape[0], dtype=np.float64)
    for j, e in enumerate(ids):
        ex = experts[int(e)]
        routed += w[j] * expert_down(ex, expert_act(ex, x))
    g = float(bf16_bits_to_f64(sgate_bits) @ x)
    shared_gated = (1.0 / (1.0 + math.exp(-g))) * expert_down(shared, expert_act(shared, x))
    out = combine(routed, shared_gated, fp16_boundary)
    return {"out": out, "ids": ids, "weights": w, "logits": logits, "routed": routed,
            "shared_gated": shared_gated, "gate": g}


def moe_prefill(X, router_bits, sgate_bits, shared, experts, top_k: int,
                fp16_boundary: bool = False, router_is_bf16_bits: bool = True, elem_scale_bits=None,
                expert_scale=None):
    """A chunk of M tokens through the routed MoE layer.

    "src/real_forward.rs", the forward state's switch for running a chunk's routed half as
    one batched dispatch pair over a route list: its output is byte-identical to running
    the tokens one at a time. So the batched call is defined as the decode call applied to
    each row of X independently. Returns dict(out [M, hidden], ids [M, k], weights [M, k]).
    """
    rows = [moe_decode(x, router_bits, sgate_bits, shared, experts, top_k, fp16_boundary,
                       router_is_bf16_bits, elem_scale_bits, expert_scale) for x in np.asarray(X)]
    return {"out": np.stack([r["out"] for r in rows]), "ids": np.stack([r["ids"] for r in rows]),
            "weights": np.stack([r["weights"] for r in rows]),
            "logits": np.stack([r["logits"] for r in rows])}

