"""Pins of the whole-layer composition oracle (oracle/layer.py) against closed forms.

Weights are chosen so that every step has a hand value: zero INT4 maps (codes 8, bias -8 s) give
exact zeros, so the low-rank read gives lo = silu(0) = 0, u = sigmoid(0) = 1/2 and
inject_w = 2 sigmoid(0) = 1; the stand-in sublayer can be the exact identity (codes 9 on the
diagonal, scale 1, bias -8); a zero router and zero experts give an MoE output of exactly 0.
"""
import numpy as np

import oracle
import synth

C, H, R, E, INTER = 4, 128, 64, 8, 64
ONE, MINUS8 = 0x3F80, 0xC100        # bf16 1.0 and -8.0


def const_int4(rows, cols, diag=False):
    q = np.full((rows, cols), 8, np.uint8)
    if diag:
        np.fill_diagonal(q, 9)
    g = cols // 64
    return synth.Int4Tensor(q=q, s_bits=np.full((rows, g), ONE, np.uint16), b_bits=np.full((rows, g), MINUS8, np.uint16))


def zero_hc(inject=True):
    return {"gamma_bits": np.full(C * H, ONE, np.uint16), "down": const_int4(R, C * H),
            "up": const_int4(C * H, R), "inject": const_int4(C, C * H) if inject else None}


def zero_moe():
    z = lambda: {"gate": const_int4(INTER, H), "up": const_int4(INTER, H), "down": const_int4(H, INTER)}
    return {"router_bits": np.zeros((E, H), np.uint16), "sgate_bits": np.zeros(H, np.uint16),
            "shared": z(), "experts": [z() for _ in range(E)], "top_k": 2}


def f16(v):
    return np.asarray(v, np.float64).astype(np.float16).astype(np.float64)


def half_normed(v):
    """mixed of a read with gamma 1 and zero low-rank maps over C identical streams: u = 1/2, so
    mixed = mean over streams of v_c / rms(v_c) / 2."""
    s = np.asarray(v, np.float64).reshape(C, H)
    n = s / np.sqrt((s * s).mean(axis=1, keepdims=True) + 1e-6)
    return (0.5 * n).mean(axis=0)


def x0():
    return synth.normal_f16(np.random.default_rng(81), (H,)).astype(np.float64)


def test_zero_sublayers_keep_the_replicated_residual():
    x = x0()
    layer = {"attn": zero_hc(), "stub": const_int4(H, H), "mlp": zero_hc(), "moe": zero_moe()}
    r = oracle.decode_layers(x, [layer], zero_hc(inject=False), C, H)
    assert np.array_equal(r["hidden"], np.tile(x, C))
    assert np.array_equal(r["mixed"], f16(half_normed(np.tile(x, C))))
    assert list(r["ids"][0]) == [0, 1]                  # all logits 0: the lowest indices


def test_identity_stand_in_injects_into_the_raw_stream():
    """out = mixed = x / rms(x) / 2 (rounded), inject weight 1: every stream becomes
    f16(x + out). Injecting into the normed stream instead would give x/rms(x) + out."""
    x = x0()
    layer = {"attn": zero_hc(), "stub": const_int4(H, H, diag=True), "mlp": zero_hc(), "moe": zero_moe()}
    r = oracle.decode_layers(x, [layer], zero_hc(inject=False), C, H)
    out = f16(half_normed(np.tile(x, C)))
    want = f16(x + out)
    assert np.array_equal(r["hidden"], np.tile(want, C))
    assert np.array_equal(r["mixed"], f16(half_normed(np.tile(want, C))))
    wrong = f16(x / np.sqrt((x * x).mean() + 1e-6) + out)
    assert not np.allclose(want, wrong)


def test_two_identity_layers_compose():
    x = x0()
    layer = {"attn": zero_hc(), "stub": const_int4(H, H, diag=True), "mlp": zero_hc(), "moe": zero_moe()}
    r = oracle.decode_layers(x, [layer, layer], zero_hc(inject=False), C, H)
    v = x
    for _ in range(2):
        v = f16(v + f16(half_normed(np.tile(v, C))))
    assert np.array_equal(r["hidden"], np.tile(v, C))
