"""GPU: the router variants through decodehp_moe_decode_ex / decodehp_moe_prefill_ex -- INT8
router codes with a per-element effective scale, a per-expert weight scale, and top-k up to 10.

Bars:
  * against the fp64 oracle (oracle.moe_decode with the same codes and scales): ids exact (order
    included), weights and output within |d| <= 1e-3 + 1e-2 |oracle|;
  * the batched call against decode calls of the same rows: bit for bit;
  * unit scales and NULL scales against the plain entry points: bit for bit (a product by 1.0
    is exact, so the kernels' arithmetic is the same sequence).
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


class Layer:
    """One MoE layer on the device; the router is the INT8 variant (codes, elem_scale,
    expert_scale), or the bf16/fp32 router of d, each with or without the scales."""

    def __init__(self, d, v=None, kind="i8", elem=True, expert=True):
        ex = d["experts"]
        self.d, self.v, self.kind = d, v, kind
        self.gate = hca.Int4Experts.from_logical([e["gate"] for e in ex])
        self.up = hca.Int4Experts.from_logical([e["up"] for e in ex])
        self.down = hca.Int4Experts.from_logical([e["down"] for e in ex])
        self.sg, self.su, self.sd = (dev_int4(d["shared"][k]) for k in ("gate", "up", "down"))
        self.sgate = hca.bf16_bits_to_tensor(d["sgate_bits"]).cuda()
        if kind == "i8":
            w = torch.from_numpy(v["codes"]).cuda()
        elif kind == "f32":
            w = torch.from_numpy(oracle.bf16_bits_to_f64(d["router_bits"]).astype(np.float32)).cuda()
        else:
            w = hca.bf16_bits_to_tensor(d["router_bits"]).cuda()
        self.elem_bits = v["elem_scale_bits"] if (v is not None and elem) else None
        self.expert_scale = v["expert_scale"] if (v is not None and expert) else None
        self.router = hca.Router(w, hca.bf16_bits_to_tensor(self.elem_bits).cuda() if self.elem_bits is not None
                                 else None,
                                 torch.from_numpy(self.expert_scale).cuda() if self.expert_scale is not None else None)
        self.plain = w

    def args(self, router, top_k):
        return (router, self.sgate, self.gate, self.up, self.down, self.sg, self.su, self.sd, top_k)

    def decode(self, x, top_k, router=None):
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        out, ids, w = hca.moe_decode(xd, *self.args(router if router is not None else self.router, top_k))
        torch.cuda.synchronize()
        return out.cpu(), ids.cpu().numpy(), w.cpu()

    def prefill(self, X, top_k):
        xd = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        out, ids, w = hca.moe_prefill(xd, *self.args(self.router, top_k))
        torch.cuda.synchronize()
        return out.cpu(), ids.cpu().numpy(), w.cpu()

    def oracle(self, x, top_k):
        if self.kind == "i8":
            r, is_bits = self.v["codes"], False
        elif self.kind == "f32":
            r, is_bits = oracle.bf16_bits_to_f64(self.d["router_bits"]).astype(np.float32), False
        else:
            r, is_bits = self.d["router_bits"], True
        return oracle.moe_decode(x, r, self.d["sgate_bits"], self.d["shared"], self.d["experts"], top_k,
                                 router_is_bf16_bits=is_bits, elem_scale_bits=self.elem_bits,
                                 expert_scale=self.expert_scale)


def check(layer, x, top_k, got=None, what="variant"):
    out, ids, w = got if got is not None else layer.decode(x, top_k)
    ref = layer.oracle(x, top_k)
    assert list(ids) == list(ref["ids"]), (what, list(ids), list(ref["ids"]))
    assert_within_tol(w.numpy(), ref["weights"], f"{what} weights")
    assert_within_tol(out.float().numpy(), ref["out"], f"{what} out")
    if layer.expert_scale is None:
        assert abs(float(w.double().sum()) - 1.0) < 1e-5
    return ref


def bits_equal(a, b):
    oa, ia, wa = a
    ob, ib, wb = b
    return (np.array_equal(ia, ib) and torch.equal(oa.view(torch.int16), ob.view(torch.int16))
            and torch.equal(wa.view(torch.int32), wb.view(torch.int32)))


@pytest.fixture(scope="module")
def full():
    say("router variants: E=256 hidden=2560 inter=512 (generating 256 experts), INT8 router + scales")
    d = synth.moe_workload(0)
    v = synth.router_variant(0, 256, 2560)
    X = np.concatenate([d["x"][None], synth.moe_x_ring(0, 127)])
    return d, v, X


@pytest.mark.parametrize("top_k", [8, 10])
def test_int8_scaled_router_workload(full, top_k):
    d, v, X = full
    L = Layer(d, v)
    for i in (0, 1, 2):
        say(f"int8 router + scales E=256 k={top_k} token {i}")
        check(L, X[i], top_k, what=f"i8 k{top_k} t{i}")


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_float_router_with_scales(full, kind):
    d, v, X = full
    say(f"{kind} router + elem and expert scales E=256 k=8")
    L = Layer(d, v, kind=kind)
    check(L, X[3], 8, what=f"{kind} scaled")


def test_top10_plain_bf16_router(full):
    d, v, X = full
    say("bf16 router, no scales, k=10, plain entry point")
    L = Layer(d, None, kind="bf16")
    got = L.decode(X[4], 10, router=L.plain)
    ref = check(L, X[4], 10, got=got, what="bf16 k10")
    assert len(ref["ids"]) == 10


def test_expert_scale_only_and_elem_scale_only(full):
    d, v, X = full
    for elem, expert in ((True, False), (False, True)):
        say(f"int8 router elem={elem} expert={expert} k=8")
        check(Layer(d, v, elem=elem, expert=expert), X[5], 8, what=f"elem{elem} expert{expert}")


def test_unit_and_null_scales_equal_the_plain_entry(full):
    d, v, X = full
    L = Layer(d, None, kind="bf16")
    say("bf16 router: plain vs _ex with NULL scales vs _ex with unit scales")
    plain = L.decode(X[6], 8, router=L.plain)
    null = L.decode(X[6], 8, router=hca.Router(L.plain))
    ones_e = hca.bf16_bits_to_tensor(np.full(2560, 0x3F80, np.uint16)).cuda()
    ones_x = torch.ones(256, dtype=torch.float32, device="cuda")
    unit = L.decode(X[6], 8, router=hca.Router(L.plain, ones_e, ones_x))
    assert bits_equal(plain, null) and bits_equal(plain, unit)


@pytest.mark.parametrize("top_k,m", [(10, 128), (8, 37)])
def test_prefill_ex_bitwise_vs_decode_ex(full, top_k, m):
    d, v, X = full
    L = Layer(d, v)
    say(f"prefill_ex int8 + scales m={m} k={top_k}")
    p = L.prefill(X[:m], top_k)
    for i in range(m):
        dd = L.decode(X[i], top_k)
        assert bits_equal((p[0][i], p[1][i], p[2][i]), dd), (top_k, m, i)
    for i in sorted({0, m // 2, m - 1}):
        check(L, X[i], top_k, got=(p[0][i], p[1][i], p[2][i]), what=f"prefill row {i}")


def small(seed, E, hidden, inter):
    rng = np.random.default_rng([93, seed, E, hidden, inter])
    mk = lambda r, c: synth.int4_tensor(rng, r, c)
    d = {"router_bits": synth.normal_bf16_bits(rng, (E, hidden), std=0.05),
         "sgate_bits": synth.normal_bf16_bits(rng, (hidden,), std=0.02),
         "shared": {"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)},
         "experts": [{"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)}
                     for _ in range(E)]}
    return d, synth.router_variant(seed, E, hidden), synth.normal_f16(rng, (5, hidden))


@pytest.mark.parametrize("E,hidden,inter,top_k", [(10, 512, 64, 10), (13, 512, 64, 10), (37, 1024, 128, 9),
                                                  (300, 1536, 64, 10), (1024, 512, 64, 10), (11, 4096, 1024, 10)])
def test_int8_variant_shapes(E, hidden, inter, top_k):
    say(f"int8 variant E={E} hidden={hidden} inter={inter} k={top_k}")
    d, v, X = small(0, E, hidden, inter)
    L = Layer(d, v)
    check(L, X[0], top_k, what=f"E{E}")
    p = L.prefill(X, top_k)
    for i in range(X.shape[0]):
        assert bits_equal((p[0][i], p[1][i], p[2][i]), L.decode(X[i], top_k)), (E, i)


def test_all_experts_selected_weights_are_scaled_softmax():
    """k = E = 10: every expert is selected, in logit order, and weight j is the softmax over
    all ten logits times the scale of expert ids[j]."""
    say("int8 variant k=E=10")
    d, v, X = small(1, 10, 512, 64)
    L = Layer(d, v)
    out, ids, w = L.decode(X[1], 10)
    assert sorted(ids.tolist()) == list(range(10))
    ref = check(L, X[1], 10, got=(out, ids, w), what="k=E")
    l32 = ref["logits"].astype(np.float32).astype(np.float64)
    sm = np.exp(l32 - l32.max())
    sm /= sm.sum()
    assert_within_tol(w.numpy(), sm[ids] * v["expert_scale"][ids], "k=E weights", atol=1e-6, rtol=1e-5)
