"""GPU parity: decodehp_moe_decode against the fp64 oracle.

Bar: expert ids bit-exact (order included, lowest index first on ties); weights and the fp16
output within |d| <= 1e-3 + 1e-2 |oracle| elementwise.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within_tol, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
hca = pytest.importorskip("hyper_connections_amd")


def dev_int4(t):
    return hca.Int4Weight.from_logical(t.q, t.s_bits, t.b_bits)


class DevMoe:
    def __init__(self, d, router_f32=False):
        ex = d["experts"]
        self.gate = hca.Int4Experts.from_logical([e["gate"] for e in ex])
        self.up = hca.Int4Experts.from_logical([e["up"] for e in ex])
        self.down = hca.Int4Experts.from_logical([e["down"] for e in ex])
        self.sg, self.su, self.sd = (dev_int4(d["shared"][k]) for k in ("gate", "up", "down"))
        if router_f32:
            self.router = torch.from_numpy(oracle.bf16_bits_to_f64(d["router_bits"]).astype(np.float32)).cuda()
        else:
            self.router = hca.bf16_bits_to_tensor(d["router_bits"]).cuda()
        self.sgate = hca.bf16_bits_to_tensor(d["sgate_bits"]).cuda()
        self.top_k = d["top_k"]

    def __call__(self, x, fp16_boundary=False):
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        out, ids, w = hca.moe_decode(xd, self.router, self.sgate, self.gate, self.up, self.down, self.sg, self.su,
                                     self.sd, self.top_k, fp16_boundary=fp16_boundary)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def check(d, dev, x, fp16_boundary=False, what="moe"):
    out, ids, w = dev(x, fp16_boundary)
    ref = oracle.moe_decode(x, d["router_bits"], d["sgate_bits"], d["shared"], d["experts"], d["top_k"],
                            fp16_boundary=fp16_boundary)
    assert list(ids) == list(ref["ids"]), (list(ids), list(ref["ids"]))
    assert_within_tol(w, ref["weights"], f"{what} weights")
    assert abs(float(np.sum(w, dtype=np.float64)) - 1.0) < 1e-5
    assert_within_tol(out, ref["out"], f"{what} out")
    l32 = np.sort(ref["logits"].astype(np.float32))[::-1]
    return float(l32[d["top_k"] - 1] - l32[d["top_k"]]) if len(l32) > d["top_k"] else None


@pytest.fixture(scope="module")
def full():
    say("moe workload E=256 hidden=2560 inter=512 top8 seed 0 (generating 256 experts)")
    d = synth.moe_workload(0)
    return d, DevMoe(d)


def test_moe_workload_e256(full):
    d, dev = full
    say("moe E=256 seed 0")
    gap = check(d, dev, d["x"], what="E256")
    print(f"8th-9th logit gap {gap:.4g}")


def test_moe_workload_more_tokens(full):
    d, dev = full
    xs = synth.moe_x_ring(0, 4)
    for i, x in enumerate(xs):
        say(f"moe E=256 ring token {i}")
        check(d, dev, x, what=f"token {i}")


def test_moe_fp16_boundary_mode(full):
    d, dev = full
    say("moe fp16 boundary")
    out, ids, w = dev(d["x"], fp16_boundary=True)
    ref = oracle.moe_decode(d["x"], d["router_bits"], d["sgate_bits"], d["shared"], d["experts"], d["top_k"],
                            fp16_boundary=True)
    assert list(ids) == list(ref["ids"])
    assert_within_tol(out, ref["out"], "boundary out")


def small(seed, E, hidden, inter, top_k, router_std=0.05):
    rng = np.random.default_rng([61, seed, E, hidden, inter, top_k])
    mk = lambda r, c: synth.int4_tensor(rng, r, c)
    return {"x": synth.normal_f16(rng, (hidden,)),
            "router_bits": synth.normal_bf16_bits(rng, (E, hidden), std=router_std),
            "sgate_bits": synth.normal_bf16_bits(rng, (hidden,), std=0.02),
            "shared": {"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)},
            "experts": [{"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)}
                        for _ in range(E)],
            "top_k": top_k}


@pytest.mark.parametrize("E,hidden,inter,top_k", [(16, 512, 64, 1), (16, 512, 64, 3), (16, 512, 64, 8),
                                                  (40, 1024, 128, 8), (8, 512, 192, 8), (300, 1536, 64, 5),
                                                  (1024, 512, 64, 8), (9, 4096, 1024, 2)])
def test_moe_shapes(E, hidden, inter, top_k):
    say(f"moe E={E} hidden={hidden} inter={inter} k={top_k}")
    d = small(0, E, hidden, inter, top_k)
    check(d, DevMoe(d), d["x"], what=f"E{E}")


def test_moe_fp32_router():
    say("moe fp32 router")
    d = small(1, 32, 1024, 128, 4)
    check(d, DevMoe(d, router_f32=True), d["x"], what="fp32 router")


def test_moe_top1_weight_is_one():
    say("moe top-1")
    d = small(2, 16, 512, 64, 1)
    _, _, w = DevMoe(d)(d["x"])
    assert w.tolist() == [1.0]


@pytest.mark.parametrize("case", ["pair_in_topk", "pair_straddles_cut"])
def test_moe_tie_goes_to_lowest_index(case):
    say(f"moe tie {case}")
    d = small(3, 24, 512, 64, 4, router_std=0.3)
    logits = oracle.router_logits(d["router_bits"], d["x"])
    order = list(oracle.select_topk(logits, 24))
    if case == "pair_in_topk":
        src, dst = order[1], order[-1]           # copy the 2nd best row onto the worst expert
    else:
        src, dst = order[3], order[-1]           # copy the 4th (last selected) onto a later/earlier id
    d["router_bits"][dst] = d["router_bits"][src]
    dev = DevMoe(d)
    out, ids, w = dev(d["x"])
    ref = oracle.moe_decode(d["x"], d["router_bits"], d["sgate_bits"], d["shared"], d["experts"], 4)
    assert list(ids) == list(ref["ids"])
    assert min(src, dst) in ids
    if case == "pair_in_topk":
        assert max(src, dst) in ids
        a, b = list(ids).index(min(src, dst)), list(ids).index(max(src, dst))
        assert b == a + 1 and w[a] == w[b]
    else:
        assert max(src, dst) not in ids
    assert_within_tol(out, ref["out"], "tie out")


@pytest.mark.parametrize("E,period", [(256, 3), (1024, 5), (37, 2), (64, 1)])
def test_moe_many_ties(E, period):
    """Router rows repeat with the given period, so whole classes of experts share one logit and
    the top-8 is decided by the lowest-index rule alone (ties inside one lane's group of
    consecutive experts and across lanes)."""
    say(f"moe many ties E={E} period={period}")
    d = small(5, E, 512, 64, 8)
    d["router_bits"] = d["router_bits"][np.arange(E) % period].copy()
    logits = oracle.router_logits(d["router_bits"], d["x"])
    assert len(set(logits.tolist())) <= period
    check(d, DevMoe(d), d["x"], what=f"ties E{E}/{period}")


def test_moe_identical_experts_routing_invariant():
    say("moe identical experts")
    d = small(4, 12, 512, 64, 3)
    d["experts"] = [d["experts"][0]] * 12
    dev = DevMoe(d)
    o1, i1, _ = dev(d["x"])
    d2 = dict(d)
    d2["router_bits"] = d["router_bits"][::-1].copy()
    o2, i2, _ = DevMoe(d2)(d["x"])
    assert list(i1) != list(i2)
    assert_within_tol(o1, o2, "routing invariance")


def test_moe_deterministic(full):
    d, dev = full
    say("moe determinism")
    a = dev(d["x"])
    b = dev(d["x"])
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def _rows_int4(rows, cols, entries, scales):
    """INT4 tensor, bias -8s: row r has codes 8 + m at the (col, m) pairs of entries[r], 8 (weight
    0) elsewhere, and scale scales[r] (a power of two, exact in bf16)."""
    q = np.full((rows, cols), 8, np.uint8)
    for r, pairs in enumerate(entries):
        for col, mult in pairs:
            q[r, col] = 8 + mult
    s = np.repeat(synth.to_bf16_bits(np.asarray(scales, np.float64))[:, None], cols // 64, axis=1)
    b = np.repeat(synth.to_bf16_bits(-8 * np.asarray(scales, np.float64))[:, None], cols // 64, axis=1)
    return synth.Int4Tensor(q=q, s_bits=s, b_bits=b)


def _hand_expert(hidden, inter, up_scales, down_pairs, down_scale):
    """gate rows 0..len(up_scales)-1 read x[0] at scale 1 (x[0] = 64: g = 64, silu(g) = g in
    fp32 and fp64); up row i reads x[0] at up_scales[i]; every down row adds the act entries of
    down_pairs at down_scale."""
    n = len(up_scales)
    rest = [()] * (inter - n)
    return {"gate": _rows_int4(inter, hidden, [((0, 1),)] * n + rest, [1.0] * inter),
            "up": _rows_int4(inter, hidden, [((0, 1),)] * n + rest, list(up_scales) + [1.0] * (inter - n)),
            "down": _rows_int4(hidden, inter, [tuple(down_pairs)] * hidden, [down_scale] * hidden)}


def test_moe_fp16_boundary_hand_values():
    """A layer built by hand so that the two output modes differ in the fp16 output itself.

    Routed (top-1, weight 1): act[0] = 64 * 64 * 2^-12 = 1 and act[1] = 64 * 64 * 2^-23 = 2^-11,
    summed by every down row: 1 + 2^-11, halfway between two fp16 values. Shared: act[0] = 1
    read at scale 2^-11, gated by sigmoid(0) = 1/2: 2^-12. Every step is exact in fp32.
      default:       fp16(1 + 2^-11 + 2^-12) = 1 + 2^-10 (three quarters of an ulp up)
      fp16 boundary: fp16(fp16(1 + 2^-11) + fp16(2^-12)) = fp16(1 + 2^-12) = 1 (ties to even)
    The oracle gives the same two values ("src/families/qwen4/mod.rs", section MoE)."""
    say("moe fp16 boundary hand values")
    hidden, inter, E = 512, 64, 8
    x = np.zeros(hidden, np.float16)
    x[0] = 64.0
    routed = _hand_expert(hidden, inter, [2.0 ** -12, 2.0 ** -23], [(0, 1), (1, 1)], 1.0)
    shared = _hand_expert(hidden, inter, [2.0 ** -12], [(0, 1)], 2.0 ** -11)
    zero = _hand_expert(hidden, inter, [], [], 1.0)
    d = {"x": x, "router_bits": np.zeros((E, hidden), np.uint16), "sgate_bits": np.zeros(hidden, np.uint16),
         "shared": shared, "experts": [routed] + [zero] * (E - 1), "top_k": 1}
    dev = DevMoe(d)
    for boundary, want in ((False, 1.0 + 2.0 ** -10), (True, 1.0)):
        out, ids, w = dev(x, fp16_boundary=boundary)
        ref = oracle.moe_decode(x, d["router_bits"], d["sgate_bits"], shared, d["experts"], 1, fp16_boundary=boundary)
        assert list(ids) == [0] and w.tolist() == [1.0]
        assert np.all(ref["out"].astype(np.float16) == np.float16(want))
        assert np.all(out == want), (boundary, np.unique(out))
