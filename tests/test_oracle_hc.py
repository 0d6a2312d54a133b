"""Pins for oracle.hc: grouped RMS norm, the low-rank mix with its two 1/C, and the inject."""
import math
import os

import numpy as np
import pytest

import oracle
import oracle.hc as oh
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def bf16(v):
    return synth.to_bf16_bits(v)[()]


def selector_int4(rows, cols, picks, scale):
    """Row r is `scale` at column picks[r] (None: all zero); built from codes q=9 / q=8 with b=-8s."""
    q = np.full((rows, cols), 8, np.uint8)
    for r, p in enumerate(picks):
        if p is not None:
            q[r, p] = 9
    s = np.full((rows, cols // 64), bf16(scale), np.uint16)
    b = np.full((rows, cols // 64), bf16(-8 * scale), np.uint16)
    return synth.Int4Tensor(q=q, s_bits=s, b_bits=b)


def const_raw(C, H, vals):
    return np.concatenate([np.full(H, v, np.float16) for v in vals])


def unit_gamma(C, H):
    return np.full(C * H, bf16(1.0), np.uint16)


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def silu(z):
    return z / (1.0 + math.exp(-z))


# ----------------------------------------------------------------- norm

def test_norm_constant_groups_closed_form():
    C, H = 4, 128
    vals = [0.5, -2.0, 3.0, 0.0]
    n = oracle.grouped_rmsnorm(const_raw(C, H, vals), unit_gamma(C, H), C, H)
    for c, a in enumerate(vals):
        expect = a / math.sqrt(a * a + EPS)
        assert np.all(np.abs(n[c * H:(c + 1) * H] - expect) <= 1e-15)


def test_norm_gamma_is_a_direct_scale():
    # hc.rs doc: the stored scale multiplies directly (not 1 + w).
    rng = np.random.default_rng(20)
    C, H = 2, 64
    raw = synth.normal_f16(rng, (C * H,))
    g_bits = synth.normal_bf16_bits(rng, (C * H,), mean=1.0, std=0.3)
    n1 = oracle.grouped_rmsnorm(raw, unit_gamma(C, H), C, H)
    n = oracle.grouped_rmsnorm(raw, g_bits, C, H)
    np.testing.assert_array_equal(n, n1 * oracle.bf16_bits_to_f64(g_bits))


def test_norm_groups_are_independent():
    rng = np.random.default_rng(21)
    C, H = 4, 64
    raw = synth.normal_f16(rng, (C * H,))
    n = oracle.grouped_rmsnorm(raw, unit_gamma(C, H), C, H)
    raw2 = raw.copy()
    raw2[H:2 * H] *= np.float16(8)
    n2 = oracle.grouped_rmsnorm(raw2, unit_gamma(C, H), C, H)
    assert np.array_equal(np.delete(n, range(H, 2 * H)), np.delete(n2, range(H, 2 * H)))


def test_norm_unit_rms_without_eps():
    rng = np.random.default_rng(22)
    C, H = 3, 256
    raw = synth.normal_f16(rng, (C * H,)) * np.float16(3)
    n = oracle.grouped_rmsnorm(raw, unit_gamma(C, H), C, H, eps=0.0).reshape(C, H)
    for c in range(C):
        assert abs(math.fsum(n[c] ** 2) / H - 1.0) < 1e-13


# ----------------------------------------------------------------- read

def _blocks(C, H, R, seed=23):
    rng = np.random.default_rng(seed)
    return (synth.int4_tensor(rng, R, C * H), synth.int4_tensor(rng, C * H, R), synth.int4_tensor(rng, C, C * H))


def test_zero_up_gives_half_mean_of_normed():
    # up == 0 -> u = sigmoid(0) = 1/2 everywhere -> mixed = (1/2) * mean_c normed[c, :].
    C, H, R = 4, 128, 64
    vals = [1.0, -0.5, 2.0, 0.25]
    down, _, inject = _blocks(C, H, R)
    up0 = selector_int4(C * H, R, [None] * (C * H), 0.125)
    out = oracle.hc_read(const_raw(C, H, vals), unit_gamma(C, H), down, up0, inject, C, H)
    expect = 0.5 * sum(a / math.sqrt(a * a + EPS) for a in vals) / C
    np.testing.assert_allclose(out["mixed"], expect, rtol=0, atol=1e-15)


def test_zero_inject_gives_one():
    C, H, R = 4, 64, 64
    down, up, _ = _blocks(C, H, R)
    rng = np.random.default_rng(24)
    raw = synth.normal_f16(rng, (C * H,))
    inj0 = selector_int4(C, C * H, [None] * C, 0.25)
    out = oracle.hc_read(raw, unit_gamma(C, H), down, up, inj0, C, H)
    assert np.all(out["inject_w"] == 1.0)


def test_selector_weights_fix_both_divisions_and_the_mean():
    # down row r reads normed[j_r]; up row (c*H + h) reads lo[h % R]; inject row c reads normed[c*H].
    C, H, R = 4, 128, 64
    rng = np.random.default_rng(25)
    raw = synth.normal_f16(rng, (C * H,))
    g_bits = synth.normal_bf16_bits(rng, (C * H,), mean=1.0, std=0.02)
    jr = [int(v) for v in rng.integers(0, C * H, size=R)]
    sd, su, si = 2.0, 4.0, 8.0
    down = selector_int4(R, C * H, jr, sd)
    up = selector_int4(C * H, R, [i % H % R for i in range(C * H)], su)
    inject = selector_int4(C, C * H, [c * H for c in range(C)], si)
    out = oracle.hc_read(raw, g_bits, down, up, inject, C, H)
    # normed by the (separately pinned) norm
    n = oracle.grouped_rmsnorm(raw, g_bits, C, H)
    lo = [silu(sd * n[j] / C) for j in jr]
    for h in range(H):
        expect = sum(sig(su * lo[h % R]) * n[c * H + h] for c in range(C)) / C
        assert abs(out["mixed"][h] - expect) < 1e-14
    for c in range(C):
        assert abs(out["inject_w"][c] - 2 * sig(si * n[c * H] / C)) < 1e-15


def test_final_mixer_has_no_inject():
    C, H, R = 2, 64, 64
    down, up, _ = _blocks(C, H, R)
    rng = np.random.default_rng(26)
    out = oracle.hc_read(synth.normal_f16(rng, (C * H,)), unit_gamma(C, H), down, up, None, C, H)
    assert out["inject_w"] is None and out["mixed"].shape == (H,)


# ----------------------------------------------------------------- inject

def test_inject_golden_c2():
    with open(os.path.join(GOLDEN, "hc_inject_c2.txt")) as f:
        d = {ln.split()[0]: [float(v) for v in ln.split()[1:]] for ln in f if ln.strip() and not ln.startswith("#")}
    got = oracle.hc_inject(d["raw"], d["out"], d["inject_w"], 2, 3)
    assert list(got) == d["hidden"]


def test_inject_c1_is_plain_residual_add():
    rng = np.random.default_rng(27)
    raw = synth.normal_f16(rng, (256,))
    out = synth.normal_f16(rng, (256,))
    np.testing.assert_array_equal(oracle.hc_inject(raw, out, [1.0], 1, 256),
                                  raw.astype(np.float64) + out.astype(np.float64))


def test_inject_zero_weights_leave_raw():
    rng = np.random.default_rng(28)
    raw = synth.normal_f16(rng, (4 * 64,))
    out = synth.normal_f16(rng, (64,))
    np.testing.assert_array_equal(oracle.hc_inject(raw, out, [0.0] * 4, 4, 64), raw.astype(np.float64))


# ----------------------------------------------------------------- planted mistakes

def _mutant_read(third_div=False, sum_mix=False, no_inject_div=False, no_double=False, one_plus_gamma=False):
    def read(raw, gamma_bits, down, up, inject, C, H, eps=oh.RMS_EPS):
        g = gamma_bits
        if one_plus_gamma:
            g = synth.to_bf16_bits(1.0 + oracle.bf16_bits_to_f64(gamma_bits))
        n = oracle.grouped_rmsnorm(raw, g, C, H, eps)
        lo = oh._silu(oracle.dequant_gemv(down.q, down.s_bits, down.b_bits, n) / C)
        pre = oracle.dequant_gemv(up.q, up.s_bits, up.b_bits, lo)
        u = oh._sigmoid(pre / C if third_div else pre)
        prod = u.reshape(C, H) * n.reshape(C, H)
        mixed = prod.sum(axis=0) if sum_mix else prod.mean(axis=0)
        iw = None
        if inject is not None:
            z = oracle.dequant_gemv(inject.q, inject.s_bits, inject.b_bits, n)
            z = z if no_inject_div else z / C
            iw = (1.0 if no_double else 2.0) * oh._sigmoid(z)
        return {"mixed": mixed, "inject_w": iw}
    return read


READ_PINS = (test_zero_up_gives_half_mean_of_normed, test_zero_inject_gives_one,
             test_selector_weights_fix_both_divisions_and_the_mean)


@pytest.mark.parametrize("kind", ["third_div", "sum_mix", "no_inject_div", "no_double", "one_plus_gamma"])
def test_planted_read_mistakes_fail_a_pin(monkeypatch, kind):
    monkeypatch.setattr(oracle, "hc_read", _mutant_read(**{kind: True}))
    failures = 0
    for pin in READ_PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_planted_inject_into_normed_fails(monkeypatch):
    # THE INJECTION TRAP: adding the sublayer output to the normed stream is a different model.
    def bad(raw, out, inject_w, C, H):
        n = oracle.grouped_rmsnorm(raw, np.full(C * H, bf16(1.0), np.uint16), C, H)
        return n + (np.asarray(out, np.float64)[None, :] * np.asarray(inject_w, np.float64)[:, None]).reshape(-1)
    monkeypatch.setattr(oracle, "hc_inject", bad)
    failures = 0
    for pin in (test_inject_golden_c2, test_inject_c1_is_plain_residual_add, test_inject_zero_weights_leave_raw):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures == 3


def test_planted_transposed_inject_layout_fails(monkeypatch):
    def bad(raw, out, inject_w, C, H):    # h-major instead of stream-major
        r = np.asarray(raw, np.float64).reshape(H, C)
        return (r + np.asarray(out, np.float64)[:, None] * np.asarray(inject_w, np.float64)[None, :]).reshape(-1)
    monkeypatch.setattr(oracle, "hc_inject", bad)
    with pytest.raises(AssertionError):
        test_inject_golden_c2()


def test_hc_read_batched_rows_are_independent_reads():
    """A chunk's read is the per-token read on every row: one row equals hc_read, reordering the
    rows reorders the outputs, and a row does not depend on the other rows."""
    rng = np.random.default_rng(77)
    C, H, R = 2, 128, 64
    blk = synth.hc_block(rng, C, H, R)
    rows = synth.normal_f16(rng, (4, C * H))
    b = oracle.hc_read_batched(rows, blk["gamma_bits"], blk["down"], blk["up"], blk["inject"], C, H)
    one = oracle.hc_read(rows[2], blk["gamma_bits"], blk["down"], blk["up"], blk["inject"], C, H)
    assert np.array_equal(b["mixed"][2], one["mixed"]) and np.array_equal(b["inject_w"][2], one["inject_w"])
    perm = [3, 1, 0, 2]
    p = oracle.hc_read_batched(rows[perm], blk["gamma_bits"], blk["down"], blk["up"], blk["inject"], C, H)
    assert np.array_equal(p["mixed"], b["mixed"][perm])
    mixer = oracle.hc_read_batched(rows, blk["gamma_bits"], blk["down"], blk["up"], None, C, H)
    assert mixer["inject_w"] is None and np.array_equal(mixer["mixed"], b["mixed"])


def test_hc_inject_batched_uses_each_rows_gate():
    C, H = 2, 64
    raw = np.zeros((2, C * H))
    out = np.ones((2, H))
    w = np.array([[1.0, 2.0], [3.0, 4.0]])
    got = oracle.hc_inject_batched(raw, out, w, C, H)
    assert np.array_equal(got[0], np.repeat([1.0, 2.0], H)) and np.array_equal(got[1], np.repeat([3.0, 4.0], H))
