"""Pins of the router variants in oracle.moe: the per-element router scale, INT8 router codes,
the per-expert weight scale, and top-k up to 10 ("src/families/qwen/state.rs", struct
RealQwenState, router_ones / per_expert_ones; "src/families/qwen4/mod.rs", section "MoE").

Each pin has a value fixed by the definition, not by the oracle's own formula:
  * a one-hot per-element scale turns the logits into one column of R times x[n];
  * a power-of-two per-element scale multiplies every logit exactly, so the selection stays
    and the weights become the softmax of the scaled logits (two-expert closed form);
  * INT8 one-hot rows give signed values of x, the code -128 included;
  * the per-expert scale of a top-1 route is that route's weight, and it never moves the
    selection;
  * k = 10 against an exhaustive subset search.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import oracle.moe as om
import synth


def bf16(v):
    return int(synth.to_bf16_bits(np.array([v], np.float64))[0])


def tiny(seed, E=12, hidden=128, inter=64):
    rng = np.random.default_rng([91, seed])
    mk = lambda r, c: synth.int4_tensor(rng, r, c)
    x = synth.normal_f16(rng, (hidden,))
    router = synth.normal_bf16_bits(rng, (E, hidden), std=0.1)
    sgate = synth.normal_bf16_bits(rng, (hidden,), std=0.02)
    shared = {"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)}
    experts = [{"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)} for _ in range(E)]
    return x, router, sgate, shared, experts


def test_one_hot_elem_scale_selects_a_column():
    x, router, *_ = tiny(0)
    n0 = 37
    es = np.zeros(x.shape[0], np.uint16)
    es[n0] = bf16(1.0)
    got = oracle.router_logits(router, x, elem_scale_bits=es)
    col = oracle.bf16_bits_to_f64(router[:, n0]) * float(x[n0])
    assert np.array_equal(got, col)
    # scaled per input element n, not per expert: the same scale laid along experts differs
    assert not np.allclose(got, oracle.router_logits(router, x) * (np.arange(len(got)) == n0))


def test_power_of_two_elem_scale_scales_logits_exactly():
    x, router, *_ = tiny(1)
    es = np.full(x.shape[0], bf16(4.0), np.uint16)
    base = oracle.router_logits(router, x)
    got = oracle.router_logits(router, x, elem_scale_bits=es)
    assert np.array_equal(got, 4.0 * base)


def test_scaled_weights_two_expert_closed_form():
    x, router, sgate, shared, experts = tiny(2, E=2)
    es = np.full(x.shape[0], bf16(0.5), np.uint16)
    r = oracle.moe_decode(x, router, sgate, shared, experts, 2, elem_scale_bits=es)
    l = oracle.bf16_bits_to_f64(router) @ x.astype(np.float64)
    l32 = (0.5 * l).astype(np.float32).astype(np.float64)
    hi = int(np.argmax(l32)) if l32[0] != l32[1] else 0
    w_hi = 1.0 / (1.0 + math.exp(-abs(l32[0] - l32[1])))
    assert int(r["ids"][0]) == hi
    np.testing.assert_allclose(r["weights"], [w_hi, 1.0 - w_hi], rtol=1e-14, atol=0)


def test_int8_one_hot_rows_give_signed_x():
    hidden, E = 64, 6
    x = synth.normal_f16(np.random.default_rng(5), (hidden,)).astype(np.float64)
    codes = np.zeros((E, hidden), np.int8)
    cols = [3, 9, 20, 41, 50, 63]
    mult = [1, -1, 127, -128, 2, -3]
    for e in range(E):
        codes[e, cols[e]] = mult[e]
    got = oracle.router_logits(codes, x, router_is_bf16_bits=False)
    assert np.array_equal(got, np.array([mult[e] * x[cols[e]] for e in range(E)]))
    assert got[3] == -128.0 * x[cols[3]]        # the code -128 is negative, not 128


def test_int8_router_with_elem_scale_is_scaled_codes():
    """INT8 codes q with a per-element scale s equal, logit for logit, a float router of q
    with x replaced by s*x; with s a power of two per element the products are exact."""
    rng = np.random.default_rng(6)
    E, hidden = 10, 128
    x = synth.normal_f16(rng, (hidden,)).astype(np.float64)
    q = rng.integers(-127, 128, size=(E, hidden)).astype(np.int8)
    pw = rng.integers(-12, -6, size=hidden)
    es = synth.to_bf16_bits(np.ldexp(1.0, pw))
    got = oracle.router_logits(q, x, router_is_bf16_bits=False, elem_scale_bits=es)
    want = np.array([math.fsum(int(q[e, n]) * math.ldexp(x[n], int(pw[n])) for n in range(hidden))
                     for e in range(E)])
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_expert_scale_top1_is_the_weight():
    x, router, sgate, shared, experts = tiny(3)
    scale = np.linspace(0.25, 3.0, len(experts)).astype(np.float32)
    r = oracle.moe_decode(x, router, sgate, shared, experts, 1, expert_scale=scale)
    e = int(r["ids"][0])
    assert r["weights"][0] == np.float64(scale[e])
    assert e == int(np.argmax(oracle.router_logits(router, x).astype(np.float32)))


def test_expert_scale_never_moves_selection_and_scales_each_weight():
    x, router, sgate, shared, experts = tiny(4)
    k = 5
    plain = oracle.moe_decode(x, router, sgate, shared, experts, k)
    scale = (10.0 ** np.arange(-3, len(experts) - 3)).astype(np.float32)   # large spread
    r = oracle.moe_decode(x, router, sgate, shared, experts, k, expert_scale=scale)
    assert list(r["ids"]) == list(plain["ids"])
    np.testing.assert_allclose(r["weights"], plain["weights"] * scale[plain["ids"]].astype(np.float64),
                               rtol=1e-15, atol=0)
    # the weighted sum uses the scaled weight of each expert
    routed = sum(r["weights"][j] * oracle.expert_down(experts[e], oracle.expert_act(experts[e], x))
                 for j, e in enumerate(r["ids"]))
    np.testing.assert_allclose(r["routed"], routed, rtol=1e-13, atol=1e-13)


def test_unit_scales_equal_the_plain_router():
    x, router, sgate, shared, experts = tiny(7)
    ones_e = np.full(x.shape[0], bf16(1.0), np.uint16)
    ones_x = np.ones(len(experts), np.float32)
    a = oracle.moe_decode(x, router, sgate, shared, experts, 4)
    b = oracle.moe_decode(x, router, sgate, shared, experts, 4, elem_scale_bits=ones_e, expert_scale=ones_x)
    assert list(a["ids"]) == list(b["ids"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["weights"], b["weights"])


@pytest.mark.parametrize("seed", range(4))
def test_top10_matches_exhaustive_subset_search(seed):
    rng = np.random.default_rng([92, seed])
    E, k = 13, 10
    logits = rng.integers(-3, 4, size=E).astype(np.float64) if seed % 2 else rng.normal(size=E)
    best = None
    for sub in itertools.combinations(range(E), k):
        key = (-math.fsum(logits[list(sub)]), sub)
        best = key if best is None or key < best else best
    ids = oracle.select_topk(logits, k)
    assert sorted(ids) == list(best[1])
    vals = logits[ids]
    assert all(vals[i] >= vals[i + 1] for i in range(k - 1))


def test_prefill_rows_are_scaled_decodes():
    x, router, sgate, shared, experts = tiny(8)
    X = synth.normal_f16(np.random.default_rng(8), (3, x.shape[0]))
    es = synth.to_bf16_bits(np.random.default_rng(9).uniform(0.5, 1.5, size=x.shape[0]))
    sc = np.random.default_rng(10).uniform(0.5, 1.5, size=len(experts)).astype(np.float32)
    p = oracle.moe_prefill(X, router, sgate, shared, experts, 10, elem_scale_bits=es, expert_scale=sc)
    for i in range(3):
        d = oracle.moe_decode(X[i], router, sgate, shared, experts, 10, elem_scale_bits=es, expert_scale=sc)
        assert np.array_equal(p["out"][i], d["out"]) and list(p["ids"][i]) == list(d["ids"])


# ----------------------------------------------------------------- planted mistakes

def _pins():
    return (test_one_hot_elem_scale_selects_a_column, test_power_of_two_elem_scale_scales_logits_exactly,
            test_scaled_weights_two_expert_closed_form, test_int8_router_with_elem_scale_is_scaled_codes,
            test_expert_scale_top1_is_the_weight, test_expert_scale_never_moves_selection_and_scales_each_weight)


def _failures():
    n = 0
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            n += 1
    return n


def test_pins_pass_unplanted():
    assert _failures() == 0


def test_planted_scale_indexed_by_expert_fails(monkeypatch):
    real = om.router_logits

    def bad(router, x, router_is_bf16_bits=True, elem_scale_bits=None):
        l = real(router, x, router_is_bf16_bits)
        if elem_scale_bits is None:
            return l
        s = oracle.bf16_bits_to_f64(elem_scale_bits)[: l.shape[0]]
        return l * s
    monkeypatch.setattr(om, "router_logits", bad)
    monkeypatch.setattr(oracle, "router_logits", bad)
    assert _failures() >= 1


def test_planted_expert_scale_before_selection_fails(monkeypatch):
    real_sel = om.select_topk
    state = {}

    def bad_decode(x, router_bits, sgate_bits, shared, experts, top_k, fp16_boundary=False,
                   router_is_bf16_bits=True, elem_scale_bits=None, expert_scale=None):
        logits = om.router_logits(router_bits, x, router_is_bf16_bits, elem_scale_bits)
        if expert_scale is not None:
            logits = logits * np.asarray(expert_scale, np.float64)        # scale folded into the logits
        ids = real_sel(logits, top_k)
        w = om.softmax_selected(logits, ids)
        routed = sum(w[j] * om.expert_down(experts[int(e)], om.expert_act(experts[int(e)], x))
                     for j, e in enumerate(ids))
        state["n"] = state.get("n", 0) + 1
        return {"out": routed, "ids": ids, "weights": w, "logits": logits, "routed": routed,
                "shared_gated": 0 * routed, "gate": 0.0}
    monkeypatch.setattr(om, "moe_decode", bad_decode)
    monkeypatch.setattr(oracle, "moe_decode", bad_decode)
    assert _failures() >= 1


def test_planted_unsigned_int8_fails(monkeypatch):
    real = om.router_logits

    def bad(router, x, router_is_bf16_bits=True, elem_scale_bits=None):
        r = np.asarray(router)
        if r.dtype == np.int8:
            r = r.view(np.uint8)
        return real(r, x, router_is_bf16_bits, elem_scale_bits)
    monkeypatch.setattr(om, "router_logits", bad)
    monkeypatch.setattr(oracle, "router_logits", bad)
    assert _failures() >= 1
