"""Pins for oracle.int4 / oracle.gemv against things other than the oracle itself.

Each pin is chosen so a plausible mistake fails it: a dropped bias, a flipped sign, a
group indexed by k % groups instead of k // 64, a transposed weight, a lost column.
"""
import itertools
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_scalar(bits: int) -> float:
    """Independent bf16 decoder: place the 16 bits on top of an fp32 word (struct, not numpy)."""
    return struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))[0]


def tiny_int4(rng, n, k):
    return synth.int4_tensor(rng, n, k)


# ----------------------------------------------------------------- dequantization

def test_dequant_code_table_golden():
    rows = []
    with open(os.path.join(GOLDEN, "dequant_codes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, b, q, w = line.split()
            rows.append((int(s, 16), int(b, 16), int(q), float(w)))
    assert len(rows) == 25
    for s, b, q, w in rows:
        got = oracle.dequant(np.full((1, 64), q, np.uint8), np.array([[s]], np.uint16),
                             np.array([[b]], np.uint16))
        assert np.all(got == w), (s, b, q, got[0, 0], w)


def test_dequant_group_index_selector():
    # Scale 2^-(g+n) and bias g+10n per (row n, group g): every element names its own group and row.
    rng = np.random.default_rng(1)
    n, k = 3, 256
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    s = np.array([[synth.to_bf16_bits(2.0 ** -(g + r))[()] for g in range(4)] for r in range(n)], np.uint16)
    b = np.array([[synth.to_bf16_bits(g + 10 * r)[()] for g in range(4)] for r in range(n)], np.uint16)
    W = oracle.dequant(q, s, b)
    for r in range(n):
        for kk in range(k):
            g = kk // 64
            assert W[r, kk] == q[r, kk] * 2.0 ** -(g + r) + (g + 10 * r)


def test_dequant_zero_point_midcode():
    # b = -8 s and q = 8 gives exactly zero for any scale.
    rng = np.random.default_rng(2)
    t = synth.int4_tensor(rng, 4, 128)
    W = oracle.dequant(np.full((4, 128), 8, np.uint8), t.s_bits, t.b_bits)
    assert np.all(W == 0.0)


def test_dequant_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.dequant(np.zeros((1, 65), np.uint8), np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))
    with pytest.raises(ValueError):
        oracle.dequant(np.full((1, 64), 16, np.uint8), np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))


# ----------------------------------------------------------------- GEMV

def test_gemv_unit_vectors_give_columns():
    # x = e_j returns column j of W, built element by element from the scalar decoder.
    rng = np.random.default_rng(3)
    n, k = 5, 192
    t = tiny_int4(rng, n, k)
    for j in range(k):
        x = np.zeros(k)
        x[j] = 1.0
        y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x)
        for r in range(n):
            expect = int(t.q[r, j]) * bf16_scalar(t.s_bits[r, j // 64]) + bf16_scalar(t.b_bits[r, j // 64])
            assert y[r] == expect


def test_gemv_exact_rational_brute_force():
    # Dyadic inputs: every product and partial sum is exact in fp64, so the oracle must
    # equal the exact rational sum bit for bit.
    rng = np.random.default_rng(4)
    n, k = 3, 128
    t = tiny_int4(rng, n, k)
    x = (rng.integers(-32, 33, size=k) / 8.0)
    y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x)
    for r in range(n):
        acc = Fraction(0)
        for kk in range(k):
            s = Fraction(bf16_scalar(t.s_bits[r, kk // 64]))
            b = Fraction(bf16_scalar(t.b_bits[r, kk // 64]))
            acc += (int(t.q[r, kk]) * s + b) * Fraction(x[kk])
        assert Fraction(y[r]) == acc


def test_gemv_fp16_inputs_near_exact():
    # Arbitrary fp16 activations: the fp64 result is within a few ulps of the exact sum.
    rng = np.random.default_rng(5)
    n, k = 4, 256
    t = tiny_int4(rng, n, k)
    x = synth.normal_f16(rng, (k,))
    y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x)
    for r in range(n):
        exact = math.fsum((int(t.q[r, kk]) * bf16_scalar(t.s_bits[r, kk // 64])
                           + bf16_scalar(t.b_bits[r, kk // 64])) * float(x[kk]) for kk in range(k))
        assert abs(y[r] - exact) <= 1e-13 * max(1.0, abs(exact))


def test_gemv_constant_codes_factored_form():
    # q == c everywhere: y[n] = sum_g (c*s[n,g] + b[n,g]) * sum_{k in g} x[k].
    rng = np.random.default_rng(6)
    n, k = 6, 320
    t = tiny_int4(rng, n, k)
    x = synth.normal_f16(rng, (k,)).astype(np.float64)
    for c in (0, 5, 15):
        q = np.full((n, k), c, np.uint8)
        y = oracle.dequant_gemv(q, t.s_bits, t.b_bits, x)
        for r in range(n):
            expect = math.fsum((c * bf16_scalar(t.s_bits[r, g]) + bf16_scalar(t.b_bits[r, g]))
                               * math.fsum(x[64 * g:64 * g + 64]) for g in range(k // 64))
            assert abs(y[r] - expect) <= 1e-12 * max(1.0, abs(expect))


def test_gemm_rows_are_independent_gemvs():
    # field batched_gemv_prefill: the M-row product equals M separate GEMVs.
    rng = np.random.default_rng(7)
    t = tiny_int4(rng, 9, 192)
    X = synth.normal_f16(rng, (5, 192))
    Y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert Y.shape == (5, 9)
    for m in range(5):
        y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X[m])
        np.testing.assert_allclose(Y[m], y, rtol=1e-13, atol=1e-13)


def test_gemv_linearity():
    rng = np.random.default_rng(8)
    t = tiny_int4(rng, 7, 128)
    x1 = rng.normal(size=128)
    x2 = rng.normal(size=128)
    y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x1 + 3 * x2)
    y1 = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x1)
    y2 = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x2)
    np.testing.assert_allclose(y, y1 + 3 * y2, rtol=1e-12, atol=1e-12)


def test_gemv_row_chunking_does_not_change_results():
    rng = np.random.default_rng(9)
    t = tiny_int4(rng, 37, 128)
    x = rng.normal(size=128)
    a = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x, row_chunk=5)
    b = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x, row_chunk=4096)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)   # BLAS may sum in another order


# ----------------------------------------------------------------- argmax

def test_argmax_planted_and_ties():
    L = np.zeros((3, 10))
    L[0, 7] = 5.0
    L[1, [2, 4, 9]] = 3.0                 # exact tie: lowest index wins
    L[2, 3] = 1.0
    L[2, 6] = 1.0 + 1e-12                 # equal after rounding to fp32: tie -> 3
    assert list(oracle.argmax_lowest(L)) == [7, 2, 3]
    assert int(oracle.argmax_lowest(L[0])) == 7


def test_argmax_brute_force_random():
    rng = np.random.default_rng(10)
    L = rng.integers(-3, 4, size=(50, 13)).astype(np.float64)   # many ties
    got = oracle.argmax_lowest(L)
    for m in range(50):
        best = max(L[m])
        assert got[m] == min(i for i in range(13) if L[m, i] == best)


# ----------------------------------------------------------------- planted mistakes

def _mutant_dequant_group_mod(q, s_bits, b_bits, group=64):
    n, k = q.shape
    s = oracle.bf16_bits_to_f64(s_bits).reshape(n, k // group)
    b = oracle.bf16_bits_to_f64(b_bits).reshape(n, k // group)
    idx = np.arange(k) % (k // group)            # wrong: k % groups instead of k // 64
    return q.astype(np.float64) * s[:, idx] + b[:, idx]


_REAL_DEQUANT = oracle.dequant


def _mutant_dequant_bias_sign(q, s_bits, b_bits, group=64):
    return _REAL_DEQUANT(q, s_bits, b_bits, group) - 2 * np.repeat(
        oracle.bf16_bits_to_f64(b_bits).reshape(q.shape[0], -1), group, axis=1)


@pytest.mark.parametrize("mutant", [_mutant_dequant_group_mod, _mutant_dequant_bias_sign])
def test_planted_dequant_mistakes_fail_a_pin(monkeypatch, mutant):
    import oracle.gemv as og
    monkeypatch.setattr(og, "dequant", mutant)
    monkeypatch.setattr(oracle, "dequant", mutant)
    failures = 0
    for pin in (test_dequant_code_table_golden, test_dequant_group_index_selector,
                test_gemv_unit_vectors_give_columns, test_gemv_constant_codes_factored_form):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_planted_transposed_gemv_fails_a_pin(monkeypatch):
    import oracle.gemv as og
    real = og.dequant_gemv

    def transposed(q, s_bits, b_bits, x, row_chunk=4096):
        W = oracle.dequant(q, s_bits, b_bits)
        x = np.asarray(x, np.float64)
        if W.shape[0] == W.shape[1]:
            return W.T @ x if x.ndim == 1 else x @ W
        return real(q, s_bits, b_bits, x, row_chunk)

    monkeypatch.setattr(oracle, "dequant_gemv", transposed)
    rng = np.random.default_rng(11)
    t = tiny_int4(rng, 128, 128)
    j = 5
    x = np.zeros(128)
    x[j] = 1.0
    y = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, x)
    expect = [int(t.q[r, j]) * bf16_scalar(t.s_bits[r, 0]) + bf16_scalar(t.b_bits[r, 0]) for r in range(128)]
    assert not np.array_equal(y, expect)
