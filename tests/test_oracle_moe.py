"""Pins for oracle.moe: selection, weights, expert FFN and the gated shared expert."""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import oracle.moe as om
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(v):
    return synth.to_bf16_bits(v)[()]


def selector_int4(rows, cols, picks, scale, rng=None):
    """INT4 tensor whose row r is `scale` at column picks[r] (or (col, mult) pairs) and 0 elsewhere.

    Built from codes: q = 8 gives 0 under b = -8s; q = 8 + m gives m*s.
    """
    q = np.full((rows, cols), 8, np.uint8)
    for r, p in enumerate(picks):
        if p is None:
            continue
        col, mult = (p, 1) if isinstance(p, (int, np.integer)) else p
        q[r, col] = 8 + mult
    s = np.full((rows, cols // 64), bf16(scale), np.uint16)
    b = np.full((rows, cols // 64), bf16(-8 * scale), np.uint16)
    return synth.Int4Tensor(q=q, s_bits=s, b_bits=b)


def zero_int4(rows, cols):
    return selector_int4(rows, cols, [None] * rows, 0.125)


# ----------------------------------------------------------------- selection

def test_topk_golden_with_ties():
    with open(os.path.join(GOLDEN, "topk_small.txt")) as f:
        d = {ln.split()[0]: ln.split()[1:] for ln in f if ln.strip() and not ln.startswith("#")}
    logits = np.array([float(v) for v in d["logits"]])
    ids = oracle.select_topk(logits, int(d["k"][0]))
    assert list(ids) == [int(v) for v in d["ids"]]
    np.testing.assert_allclose(oracle.softmax_selected(logits, ids), [float(v) for v in d["weights"]],
                               rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_exhaustive_subset_search(seed):
    # The selected set is the lexicographically smallest k-subset of maximal logit sum.
    rng = np.random.default_rng(seed)
    E, k = 9, 3
    logits = rng.integers(-4, 5, size=E).astype(np.float64) if seed % 2 else rng.normal(size=E)
    best = None
    for sub in itertools.combinations(range(E), k):
        key = (-math.fsum(logits[list(sub)]), sub)
        best = key if best is None or key < best else best
    ids = oracle.select_topk(logits, k)
    assert sorted(ids) == list(best[1])
    vals = logits[ids]
    assert all(vals[i] >= vals[i + 1] for i in range(k - 1))          # descending order


def test_topk_decides_on_fp32_logits():
    # Two logits that differ below fp32 resolution tie; the lower index wins.
    logits = np.array([1.0, 1.0 + 1e-12, 0.0])
    assert list(oracle.select_topk(logits, 1)) == [0]


def test_softmax_two_expert_closed_form():
    logits = np.array([0.3, -1.2, 2.0, 0.7])
    ids = oracle.select_topk(logits, 2)
    assert list(ids) == [2, 3]
    w = oracle.softmax_selected(logits, ids)
    l32 = logits.astype(np.float32).astype(np.float64)
    d = l32[2] - l32[3]
    assert abs(w[0] - 1.0 / (1.0 + math.exp(-d))) < 1e-15
    assert abs(w[1] - 1.0 / (1.0 + math.exp(d))) < 1e-15


def test_softmax_k1_and_sum_to_one():
    rng = np.random.default_rng(12)
    logits = rng.normal(size=64) * 3
    assert list(oracle.softmax_selected(logits, oracle.select_topk(logits, 1))) == [1.0]
    for k in (2, 8, 10):
        w = oracle.softmax_selected(logits, oracle.select_topk(logits, k))
        assert abs(math.fsum(w) - 1.0) < 1e-14
        assert np.all(np.diff(w) <= 0)


def test_softmax_order_identity_from_the_pages():
    # "src/families/qwen4/mod.rs", section MoE: softmax over all experts, then top-k,
    # then renormalize, equals top-k on raw logits then softmax over the selected set.
    rng = np.random.default_rng(13)
    logits = rng.normal(size=256) * 2
    ids = oracle.select_topk(logits, 8)
    l32 = logits.astype(np.float32).astype(np.float64)
    full = np.exp(l32) / np.exp(l32).sum()
    renorm = full[ids] / full[ids].sum()
    np.testing.assert_allclose(oracle.softmax_selected(logits, ids), renorm, rtol=1e-12)


def test_router_unit_vector_returns_column():
    rng = np.random.default_rng(14)
    R = synth.normal_bf16_bits(rng, (16, 128), std=0.02)
    x = np.zeros(128)
    x[37] = 1.0
    np.testing.assert_array_equal(oracle.router_logits(R, x), oracle.bf16_bits_to_f64(R)[:, 37])


# ----------------------------------------------------------------- expert FFN

def _selector_expert(hidden, inter, sg, su, sd, down_mult=1):
    # gate row i and up row i read x[i] (up with multiplier 2); down row h reads act[h % inter].
    return {"gate": selector_int4(inter, hidden, list(range(inter)), sg),
            "up": selector_int4(inter, hidden, [(i, 2) for i in range(inter)], su),
            "down": selector_int4(hidden, inter, [(h % inter, down_mult) for h in range(hidden)], sd)}


def test_expert_act_is_silu_gate_times_up():
    rng = np.random.default_rng(15)
    hidden, inter = 128, 64
    ex = _selector_expert(hidden, inter, 0.25, 0.0625, 0.5)
    x = synth.normal_f16(rng, (hidden,)).astype(np.float64) * 4
    act = oracle.expert_act(ex, x)
    for i in range(inter):
        g = 0.25 * x[i]
        u = 2 * 0.0625 * x[i]
        assert abs(act[i] - g / (1 + math.exp(-g)) * u) < 1e-14


def test_expert_down_selector():
    hidden, inter = 128, 64
    ex = _selector_expert(hidden, inter, 0.25, 0.0625, 0.5, down_mult=3)
    act = np.arange(inter, dtype=np.float64) - 20
    y = oracle.expert_down(ex, act)
    for h in range(hidden):
        assert y[h] == 1.5 * act[h % inter]


def _tiny_moe(seed, E=6, hidden=128, inter=64, top_k=3):
    rng = np.random.default_rng(seed)
    x = synth.normal_f16(rng, (hidden,))
    router = synth.normal_bf16_bits(rng, (E, hidden), std=0.5)
    sgate = synth.normal_bf16_bits(rng, (hidden,), std=0.1)
    mk = lambda: {"gate": synth.int4_tensor(rng, inter, hidden), "up": synth.int4_tensor(rng, inter, hidden),
                  "down": synth.int4_tensor(rng, hidden, inter)}
    return x, router, sgate, mk(), [mk() for _ in range(E)], top_k


def test_identical_experts_make_output_independent_of_routing():
    x, router, sgate, shared, experts, k = _tiny_moe(16)
    same = [experts[0]] * len(experts)
    a = oracle.moe_decode(x, router, sgate, shared, same, k)
    router2 = router[::-1].copy()
    b = oracle.moe_decode(x, router2, sgate, shared, same, k)
    assert list(a["ids"]) != list(b["ids"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)
    single = oracle.expert_down(experts[0], oracle.expert_act(experts[0], x))
    np.testing.assert_allclose(a["routed"], single, rtol=1e-12, atol=1e-12)


def test_weighted_reduce_scales_per_expert():
    # Expert e = expert 0 with its down scale multiplied by 2^e (codes unchanged), so
    # routed = (sum_j w_j 2^{ids_j}) * y0: pins that weight j multiplies expert ids_j.
    x, router, sgate, shared, experts, k = _tiny_moe(17)
    base = experts[0]
    scaled = []
    for e in range(len(experts)):
        s = oracle.bf16_bits_to_f64(base["down"].s_bits) * 2.0 ** e
        d = synth.Int4Tensor(q=base["down"].q, s_bits=synth.to_bf16_bits(s), b_bits=synth.to_bf16_bits(-8 * s))
        scaled.append({"gate": base["gate"], "up": base["up"], "down": d})
    res = oracle.moe_decode(x, router, sgate, shared, scaled, k)
    y0 = oracle.expert_down(scaled[0], oracle.expert_act(scaled[0], x))
    # weights from the separately pinned selection + softmax, not from moe_decode's own output
    logits = oracle.router_logits(router, x)
    ids = oracle.select_topk(logits, k)
    w = oracle.softmax_selected(logits, ids)
    assert list(res["ids"]) == list(ids)
    np.testing.assert_allclose(res["weights"], w, rtol=1e-15, atol=0)
    assert np.all(np.diff(res["weights"]) <= 0)
    coef = sum(w[j] * 2.0 ** int(ids[j]) for j in range(k))
    np.testing.assert_allclose(res["routed"], coef * y0, rtol=1e-12, atol=1e-12)


def test_shared_gate_zero_is_half_and_routed_zero():
    x, router, sgate, shared, experts, k = _tiny_moe(18)
    hidden, inter = 128, 64
    zero_experts = [{"gate": zero_int4(inter, hidden), "up": zero_int4(inter, hidden),
                     "down": zero_int4(hidden, inter)} for _ in experts]
    sg0 = np.zeros(hidden, np.uint16)
    res = oracle.moe_decode(x, router, sg0, shared, zero_experts, k)
    assert np.all(res["routed"] == 0.0)
    sh = oracle.expert_down(shared, oracle.expert_act(shared, x))
    np.testing.assert_array_equal(res["out"], 0.5 * sh)
    # and a nonzero gate logit g gives sigmoid(g) exactly as the logistic function
    res2 = oracle.moe_decode(x, router, sgate, shared, zero_experts, k)
    g = math.fsum(oracle.bf16_bits_to_f64(sgate) * x.astype(np.float64))
    np.testing.assert_allclose(res2["out"], sh / (1 + math.exp(-g)), rtol=1e-13, atol=1e-14)


def _int4_from_rows(rows, cols, entries, scales):
    """INT4 tensor with bias -8s everywhere: row r has codes 8 + m at the (col, m) pairs of
    entries[r] and 8 (weight 0) elsewhere, and scale scales[r] (exact in bf16)."""
    q = np.full((rows, cols), 8, np.uint8)
    for r, pairs in enumerate(entries):
        for col, mult in pairs:
            q[r, col] = 8 + mult
    s = np.repeat(np.array([[bf16(v)] for v in scales], np.uint16), cols // 64, axis=1)
    b = np.repeat(np.array([[bf16(-8 * v)] for v in scales], np.uint16), cols // 64, axis=1)
    return synth.Int4Tensor(q=q, s_bits=s, b_bits=b)


def _one_plus_2m12_expert(hidden=128, inter=64):
    """An expert whose output is 1 + 2^-12 in every element for x with x[0] = 64.

    gate rows 0 and 1 read x[0] at scale 1: g = 64, and silu(64) = 64 in float64 (exp(-64) is
    below half an ulp of 1). up row 0 reads x[0] at scale 2^-12 (u = 2^-6), up row 1 at 2^-24
    (u = 2^-18): act[0] = 1, act[1] = 2^-12, the other rows 0. Every down row adds act[0] and
    act[1] at scale 1: 1 + 2^-12, which needs 13 significant bits; fp16 keeps 11, and rounding
    to nearest even gives 1."""
    zeros = [()] * (inter - 2)
    gate = _int4_from_rows(inter, hidden, [((0, 1),), ((0, 1),)] + zeros, [1.0] * inter)
    up = _int4_from_rows(inter, hidden, [((0, 1),), ((0, 1),)] + zeros, [2.0 ** -12, 2.0 ** -24] + [1.0] * (inter - 2))
    down = _int4_from_rows(hidden, inter, [((0, 1), (1, 1))] * hidden, [1.0] * hidden)
    return {"gate": gate, "up": up, "down": down}


def _boundary_case():
    hidden, inter, E = 128, 64, 4
    x = np.zeros(hidden, np.float16)
    x[0] = 64.0
    router = np.zeros((E, hidden), np.uint16)          # all logits 0: top-1 picks expert 0, weight 1
    zero = {"gate": zero_int4(inter, hidden), "up": zero_int4(inter, hidden), "down": zero_int4(hidden, inter)}
    return x, router, _one_plus_2m12_expert(hidden, inter), zero, E


def test_fp16_boundary_casts_the_routed_sum():
    # routed = 1 + 2^-12 (the top-1 expert at weight 1), shared expert zero, gate row zero.
    x, router, ex, zero, E = _boundary_case()
    sgate = np.zeros(128, np.uint16)
    b = oracle.moe_decode(x, router, sgate, zero, [ex] + [zero] * (E - 1), 1, fp16_boundary=True)
    assert list(b["ids"]) == [0] and list(b["weights"]) == [1.0]
    assert np.all(b["out"] == 1.0)                     # fp16(1 + 2^-12) + fp16(0)
    d = oracle.moe_decode(x, router, sgate, zero, [ex] + [zero] * (E - 1), 1)
    assert np.all(d["out"] == 1.0 + 2.0 ** -12)        # default: unrounded until the end


def test_fp16_boundary_casts_the_gated_shared_half():
    # routed zero (every routed expert zero), shared expert = the 1 + 2^-12 expert, gate row 0:
    # sigmoid(0) = 1/2, so the gated shared half is 1/2 + 2^-13, which fp16 rounds to 1/2.
    x, router, ex, zero, E = _boundary_case()
    sgate = np.zeros(128, np.uint16)
    b = oracle.moe_decode(x, router, sgate, ex, [zero] * E, 1, fp16_boundary=True)
    assert np.all(b["out"] == 0.5)
    d = oracle.moe_decode(x, router, sgate, ex, [zero] * E, 1)
    assert np.all(d["out"] == 0.5 + 2.0 ** -13)


def test_fp16_boundary_rounds_each_half_not_the_sum():
    # routed = 1 + 2^-12 (fp16: 1); shared expert output 3 * 2^-11 (act[0] = 1 read with
    # multiplier 3 at scale 2^-11), gated by sigmoid(0) = 1/2: 3 * 2^-12, exact in fp16. Each
    # half rounded, then added: 1 + 3 * 2^-12; rounding the sum instead, 1 + 2^-10.
    x, router, ex, zero, E = _boundary_case()
    hidden, inter = 128, 64
    zeros = [()] * (inter - 1)
    sh = {"gate": _int4_from_rows(inter, hidden, [((0, 1),)] + zeros, [1.0] * inter),
          "up": _int4_from_rows(inter, hidden, [((0, 1),)] + zeros, [2.0 ** -12] + [1.0] * (inter - 1)),
          "down": _int4_from_rows(hidden, inter, [((0, 3),)] * hidden, [2.0 ** -11] * hidden)}
    sgate = np.zeros(128, np.uint16)
    b = oracle.moe_decode(x, router, sgate, sh, [ex] + [zero] * (E - 1), 1, fp16_boundary=True)
    assert np.all(b["out"] == 1.0 + 3 * 2.0 ** -12)
    d = oracle.moe_decode(x, router, sgate, sh, [ex] + [zero] * (E - 1), 1)
    assert np.all(d["out"] == 1.0 + 2.0 ** -10)


# ----------------------------------------------------------------- planted mistakes

def _boundary_pins():
    return (test_fp16_boundary_casts_the_routed_sum, test_fp16_boundary_casts_the_gated_shared_half,
            test_fp16_boundary_rounds_each_half_not_the_sum)


def _count_boundary_failures():
    n = 0
    for pin in _boundary_pins():
        try:
            pin()
        except AssertionError:
            n += 1
    return n


@pytest.mark.parametrize("mutant", ["no_cast", "cast_shared_only", "cast_routed_only", "cast_sum"])
def test_planted_fp16_boundary_mistakes_fail(monkeypatch, mutant):
    f16 = lambda v: np.asarray(v, np.float64).astype(np.float16).astype(np.float64)

    def bad(routed, shared_gated, fp16_boundary=False):
        r, sh = np.asarray(routed, np.float64), np.asarray(shared_gated, np.float64)
        if not fp16_boundary:
            return r + sh
        return {"no_cast": lambda: r + sh, "cast_shared_only": lambda: r + f16(sh),
                "cast_routed_only": lambda: f16(r) + sh, "cast_sum": lambda: f16(r + sh) + 0.0}[mutant]()
    monkeypatch.setattr(om, "combine", bad)
    assert _count_boundary_failures() >= 1


def _pins():
    return (test_topk_golden_with_ties, test_softmax_two_expert_closed_form, test_softmax_k1_and_sum_to_one,
            test_softmax_order_identity_from_the_pages, test_expert_act_is_silu_gate_times_up,
            test_identical_experts_make_output_independent_of_routing, test_weighted_reduce_scales_per_expert,
            test_shared_gate_zero_is_half_and_routed_zero)


def _count_failures():
    n = 0
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            n += 1
    return n


def test_planted_silu_on_up_fails(monkeypatch):
    def bad_act(expert, x):
        g = oracle.dequant_gemv(expert["gate"].q, expert["gate"].s_bits, expert["gate"].b_bits, x)
        u = oracle.dequant_gemv(expert["up"].q, expert["up"].s_bits, expert["up"].b_bits, x)
        return g * om.silu(u)
    monkeypatch.setattr(om, "expert_act", bad_act)
    monkeypatch.setattr(oracle, "expert_act", bad_act)
    assert _count_failures() >= 1


def test_planted_unnormalized_weights_fail(monkeypatch):
    def bad_softmax(logits, ids):
        l32 = np.asarray(logits, np.float64).astype(np.float32).astype(np.float64)
        return np.exp(l32[np.asarray(ids)]) / np.exp(l32).sum()      # softmax over all, no renormalization
    monkeypatch.setattr(om, "softmax_selected", bad_softmax)
    monkeypatch.setattr(oracle, "softmax_selected", bad_softmax)
    assert _count_failures() >= 1


def test_planted_reversed_weights_fail(monkeypatch):
    real = om.softmax_selected
    monkeypatch.setattr(om, "softmax_selected", lambda l, ids: real(l, ids)[::-1].copy())
    assert _count_failures() >= 1


def test_planted_highest_index_tie_break_fails(monkeypatch):
    def bad_topk(logits, k):
        l32 = np.asarray(logits, np.float64).astype(np.float32).astype(np.float64)
        return np.asarray(sorted(range(len(l32)), key=lambda e: (-l32[e], -e))[:k])
    monkeypatch.setattr(om, "select_topk", bad_topk)
    monkeypatch.setattr(oracle, "select_topk", bad_topk)
    assert _count_failures() >= 1


def _prefill_case(seed, M, E=12, hidden=128, inter=64, top_k=3):
    rng = np.random.default_rng([71, seed])
    mk = lambda r, c: synth.int4_tensor(rng, r, c)
    X = synth.normal_f16(rng, (M, hidden))
    router = synth.normal_bf16_bits(rng, (E, hidden), std=0.1)
    sgate = synth.normal_bf16_bits(rng, (hidden,), std=0.02)
    shared = {"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)}
    experts = [{"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)} for _ in range(E)]
    return X, router, sgate, shared, experts, top_k


def test_moe_prefill_one_token_is_decode():
    X, router, sgate, shared, experts, k = _prefill_case(0, 1)
    p = oracle.moe_prefill(X, router, sgate, shared, experts, k)
    d = oracle.moe_decode(X[0], router, sgate, shared, experts, k)
    assert np.array_equal(p["out"][0], d["out"])
    assert list(p["ids"][0]) == list(d["ids"]) and np.array_equal(p["weights"][0], d["weights"])


def test_moe_prefill_tokens_are_independent():
    """A chunk is M separate passes: reordering the tokens reorders the rows of every output,
    and a token's row does not change when the other tokens of the chunk change."""
    X, router, sgate, shared, experts, k = _prefill_case(1, 5)
    base = oracle.moe_prefill(X, router, sgate, shared, experts, k)
    perm = np.array([3, 0, 4, 2, 1])
    pp = oracle.moe_prefill(X[perm], router, sgate, shared, experts, k)
    assert np.array_equal(pp["out"], base["out"][perm])
    assert np.array_equal(pp["ids"], base["ids"][perm])
    X2 = X.copy()
    X2[[0, 1, 3, 4]] = synth.normal_f16(np.random.default_rng(9), (4, X.shape[1]))
    p2 = oracle.moe_prefill(X2, router, sgate, shared, experts, k)
    assert np.array_equal(p2["out"][2], base["out"][2]) and list(p2["ids"][2]) == list(base["ids"][2])
