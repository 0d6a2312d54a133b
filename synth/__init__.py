"""Seeded synthetic inputs for the decode hot path.

This module only draws random numbers and stores them in the storage formats the
path consumes (fp16, bf16 bit patterns, unsigned 4-bit codes). It holds none of the
method's arithmetic: no dequantization, no products, no norms, no routing. Both the
CPU oracle (``oracle/``) and the GPU path's tests and benchmark take their inputs
from here; neither side imports the other.

Streams. Every workload ``w`` draws from ``numpy.random.default_rng([w, seed])``
in the order its function lists; routed expert ``e`` of the MoE workload draws
from its own stream ``default_rng([2, seed, e])`` so one expert can be generated
without the other 255.

Value recipes (the decode runtime's synthetic workloads):
  * activations / residual: fp16(N(0, 1))
  * INT4 codes: uniform integers 0..15
  * per-group scale: bf16(U(0.005, 0.02)); per-group bias: bf16(-8 * scale), which
    is exact because -8 is a power of two times -1
  * router rows and the shared-expert gate row: bf16(N(0, 0.02))
  * INT8 router (the scaled-router variant): codes uniform on -127..127, per-element
    scale bf16(2.7e-4 * U(0.5, 1.5)) (logits of about the bf16 router's spread),
    per-expert scale fp32(U(0.5, 1.5))
  * hyper-connection norm weight: bf16(N(1, 0.02))
  * inject weights: fp32(U(0, 1))
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64

# Workload ids (also the first word of each stream key).
GEMV_2560 = 0
HC_C4_H2560 = 1
MOE_E256 = 2
PREFILL_M128 = 3
DECODE_LAYERS = 5
LMHEAD_151936 = 4
ROUTER_VARIANT = 6


def rng_for(workload: int, seed: int = 0, *extra: int) -> np.random.Generator:
    return np.random.default_rng([workload, seed, *extra])


# --------------------------------------------------------------------------- formats

def to_f16(a) -> np.ndarray:
    """Round to IEEE binary16 (numpy casts with round-to-nearest-even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def to_bf16_bits(a) -> np.ndarray:
    """Round to bfloat16 and return the uint16 bit patterns.

    Rounds float64 -> float32 (RNE) -> bfloat16 (RNE on the upper 16 bits).
    """
    f32 = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact). Storage helper for device upload."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Int4Tensor:
    """Logical INT4-affine tensor: codes q[N,K] in 0..15, bf16 scale/bias bits [N, K/64]."""

    q: np.ndarray        # uint8 [N, K], values 0..15
    s_bits: np.ndarray   # uint16 [N, K/64]
    b_bits: np.ndarray   # uint16 [N, K/64]

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def cols(self) -> int:
        return self.q.shape[1]


def int4_tensor(rng: np.random.Generator, rows: int, cols: int,
                scale_lo: float = 0.005, scale_hi: float = 0.02) -> Int4Tensor:
    """Codes uniform 0..15, then scales bf16(U(lo, hi)), bias bf16(-8*scale)."""
    assert cols % GROUP == 0
    q = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    s = rng.uniform(scale_lo, scale_hi, size=(rows, cols // GROUP))
    s_bits = to_bf16_bits(s)
    # -8 * bf16 value is exactly representable: flip the sign bit and add 3 to the exponent.
    b_bits = to_bf16_bits(-8.0 * bf16_bits_to_f32(s_bits).astype(np.float64))
    return Int4Tensor(q=q, s_bits=s_bits, b_bits=b_bits)


def normal_f16(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    return to_f16(rng.normal(mean, std, size=shape))


def normal_bf16_bits(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    return to_bf16_bits(rng.normal(mean, std, size=shape))


# --------------------------------------------------------------------------- workloads

def gemv_workload(seed: int = 0, n: int = 2560, k: int = 2560):
    """Single M=1 dequant GEMV: x fp16[k], weight INT4 [n x k]."""
    rng = rng_for(GEMV_2560, seed)
    x = normal_f16(rng, (k,))
    w = int4_tensor(rng, n, k)
    return {"x": x, "w": w}


def hc_workload(seed: int = 0, c: int = 4, h: int = 2560, r: int = 320):
    """Hyper-connection read + inject for one token.

    raw fp16[c*h]; hc_norm bf16[c*h]; down INT4 [r x c*h]; up INT4 [c*h x r];
    block-inject INT4 [c x c*h]; sublayer output fp16[h]; inject weights fp32[c].
    """
    rng = rng_for(HC_C4_H2560, seed)
    wide = c * h
    raw = normal_f16(rng, (wide,))
    gamma_bits = normal_bf16_bits(rng, (wide,), mean=1.0, std=0.02)
    down = int4_tensor(rng, r, wide)
    up = int4_tensor(rng, wide, r)
    inject = int4_tensor(rng, c, wide)
    out = normal_f16(rng, (h,))
    iw = rng.uniform(0.0, 1.0, size=(c,)).astype(np.float32)
    return {"raw": raw, "gamma_bits": gamma_bits, "down": down, "up": up, "inject": inject,
            "out": out, "iw": iw, "C": c, "H": h, "R": r}


def moe_expert(seed: int, e: int, hidden: int = 2560, inter: int = 512):
    """Routed expert e: gate INT4 [inter x hidden], up INT4 [inter x hidden], down INT4 [hidden x inter]."""
    rng = rng_for(MOE_E256, seed, e)
    gate = int4_tensor(rng, inter, hidden)
    up = int4_tensor(rng, inter, hidden)
    down = int4_tensor(rng, hidden, inter)
    return {"gate": gate, "up": up, "down": down}


def moe_workload(seed: int = 0, hidden: int = 2560, inter: int = 512, n_experts: int = 256,
                 top_k: int = 8, with_experts: bool = True):
    """Routed MoE decode layer at M=1.

    x fp16[hidden]; router bf16[E x hidden]; shared gate row bf16[hidden]; shared expert
    gate/up/down INT4; routed experts from their own streams (see moe_expert).
    """
    rng = rng_for(MOE_E256, seed)
    x = normal_f16(rng, (hidden,))
    router_bits = normal_bf16_bits(rng, (n_experts, hidden), std=0.02)
    sgate_bits = normal_bf16_bits(rng, (hidden,), std=0.02)
    shared = {"gate": int4_tensor(rng, inter, hidden),
              "up": int4_tensor(rng, inter, hidden),
              "down": int4_tensor(rng, hidden, inter)}
    experts = [moe_expert(seed, e, hidden, inter) for e in range(n_experts)] if with_experts else None
    return {"x": x, "router_bits": router_bits, "sgate_bits": sgate_bits, "shared": shared,
            "experts": experts, "E": n_experts, "top_k": top_k, "hidden": hidden, "inter": inter}


def router_variant(seed: int = 0, n_experts: int = 256, hidden: int = 2560) -> dict:
    """The scaled router: INT8 codes [E x hidden], bf16 per-element scale bits [hidden] and
    fp32 per-expert scales [E] (recipe in the module doc)."""
    rng = rng_for(ROUTER_VARIANT, seed, n_experts, hidden)
    codes = rng.integers(-127, 128, size=(n_experts, hidden)).astype(np.int8)
    elem_scale_bits = to_bf16_bits(2.7e-4 * rng.uniform(0.5, 1.5, size=hidden))
    expert_scale = rng.uniform(0.5, 1.5, size=n_experts).astype(np.float32)
    return {"codes": codes, "elem_scale_bits": elem_scale_bits, "expert_scale": expert_scale}


def moe_x_ring(seed: int, count: int, hidden: int = 2560) -> np.ndarray:
    """Extra activation vectors (seeds seed+1 .. seed+count) so routing varies between calls."""
    return np.stack([normal_f16(rng_for(MOE_E256, seed + 1 + i, 1_000_000), (hidden,))
                     for i in range(count)])


def prefill_workload(seed: int = 0, m: int = 128, n: int = 8192, k: int = 2560):
    """Batched chunked-prefill projection: X fp16[m x k]; packed [query; gate] INT4 [n x k]."""
    rng = rng_for(PREFILL_M128, seed)
    x = normal_f16(rng, (m, k))
    w = int4_tensor(rng, n, k)
    return {"x": x, "w": w}


def lmhead_x(seed: int = 0, m: int = 1, k: int = 2560) -> np.ndarray:
    """LM-head input rows fp16[m x k]; their own stream, so they can be drawn without the weight."""
    return normal_f16(rng_for(LMHEAD_151936, seed, m), (m, k))


def lmhead_workload(seed: int = 0, m: int = 1, n: int = 151936, k: int = 2560):
    """LM head: hidden fp16[m x k]; INT4 weight [n x k]. The weight stream does not depend on m."""
    rng = rng_for(LMHEAD_151936, seed)
    w = int4_tensor(rng, n, k)
    return {"x": lmhead_x(seed, m, k), "w": w}


def hc_block(rng: np.random.Generator, c: int, h: int, r: int, inject: bool = True) -> dict:
    """One hyper-connection read's weights: hc_norm bf16 ~N(1, 0.02) [C*H], down INT4 [R x C*H],
    up INT4 [C*H x R], inject INT4 [C x C*H] (absent for the final mixer)."""
    wide = c * h
    return {"gamma_bits": normal_bf16_bits(rng, (wide,), mean=1.0, std=0.02), "down": int4_tensor(rng, r, wide),
            "up": int4_tensor(rng, wide, r), "inject": int4_tensor(rng, c, wide) if inject else None}


def decode_layer_workload(seed: int = 0, n_layers: int = 1, c: int = 4, h: int = 2560, r: int = 320,
                          n_experts: int = 256, inter: int = 512, top_k: int = 8):
    """Whole decoder layers for one token: x fp16 [H]; per layer the attn and mlp hyper-connection
    weights, an INT4 [H x H] stand-in for the attention sublayer and an MoE layer of the MoE
    workload's distributions (router bf16 N(0, 0.02), experts INT4 from their own streams); the
    final mixer's read weights."""
    rng = rng_for(DECODE_LAYERS, seed)
    x = normal_f16(rng, (h,))
    layers = []
    for li in range(n_layers):
        lr = rng_for(DECODE_LAYERS, seed, 1 + li)
        attn, stub, mlp = hc_block(lr, c, h, r), int4_tensor(lr, h, h), hc_block(lr, c, h, r)
        moe = {"router_bits": normal_bf16_bits(lr, (n_experts, h), std=0.02),
               "sgate_bits": normal_bf16_bits(lr, (h,), std=0.02),
               "shared": {"gate": int4_tensor(lr, inter, h), "up": int4_tensor(lr, inter, h),
                          "down": int4_tensor(lr, h, inter)},
               "experts": [], "top_k": top_k}
        for e in range(n_experts):
            er = rng_for(DECODE_LAYERS, seed, 1 + li, 1 + e)
            moe["experts"].append({"gate": int4_tensor(er, inter, h), "up": int4_tensor(er, inter, h),
                                   "down": int4_tensor(er, h, inter)})
        layers.append({"attn": attn, "stub": stub, "mlp": mlp, "moe": moe})
    mixer = hc_block(rng, c, h, r, inject=False)
    return {"x": x, "layers": layers, "mixer": mixer, "C": c, "H": h, "R": r}

