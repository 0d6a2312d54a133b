"""GPU: decodehp_moe_prefill, a chunk of m tokens through one routed MoE layer.

Two bars:
  * against m decodehp_moe_decode calls on the same rows: bit for bit (fp16 output bits, ids,
    fp32 weight bits). The batched path computes every per-token value with the decode
    path's own helpers in the same order, so nothing less is accepted;
  * against the fp64 oracle (moe_prefill = moe_decode per row): ids exact, weights and output
    within |d| <= 1e-3 + 1e-2 |oracle|.
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

    def _w(self):
        return (self.router, self.sgate, self.gate, self.up, self.down, self.sg, self.su, self.sd, self.top_k)

    def prefill(self, X, fp16_boundary=False):
        xd = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        out, ids, w = hca.moe_prefill(xd, *self._w(), fp16_boundary=fp16_boundary)
        torch.cuda.synchronize()
        return out.cpu(), ids.cpu().numpy(), w.cpu()

    def decodes(self, X, fp16_boundary=False):
        outs, idss, ws = [], [], []
        for x in X:
            xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
            out, ids, w = hca.moe_decode(xd, *self._w(), fp16_boundary=fp16_boundary)
            outs.append(out.clone())
            idss.append(ids.clone())
            ws.append(w.clone())
        torch.cuda.synchronize()
        return torch.stack(outs).cpu(), torch.stack(idss).cpu().numpy(), torch.stack(ws).cpu()


def assert_bitwise(p, d, what):
    po, pi, pw = p
    do, di, dw = d
    assert np.array_equal(pi, di), f"{what}: ids differ in rows {np.nonzero((pi != di).any(1))[0][:8]}"
    bad = (po.view(torch.int16) != do.view(torch.int16)).any(1).nonzero().flatten()
    assert bad.numel() == 0, f"{what}: output bits differ in rows {bad[:8].tolist()}"
    assert torch.equal(pw.view(torch.int32), dw.view(torch.int32)), f"{what}: weight bits differ"


def check_oracle(d, X, p, rows, fp16_boundary=False, what="prefill"):
    out, ids, w = p
    for i in rows:
        ref = oracle.moe_decode(X[i], d["router_bits"], d["sgate_bits"], d["shared"], d["experts"], d["top_k"],
                                fp16_boundary=fp16_boundary)
        assert list(ids[i]) == list(ref["ids"]), (i, list(ids[i]), list(ref["ids"]))
        assert_within_tol(w[i].numpy(), ref["weights"], f"{what} row {i} weights")
        assert_within_tol(out[i].float().numpy(), ref["out"], f"{what} row {i} out")


def small(seed, E, hidden, inter, top_k, router_std=0.05):
    rng = np.random.default_rng([62, seed, E, hidden, inter, top_k])
    mk = lambda r, c: synth.int4_tensor(rng, r, c)
    return {"router_bits": synth.normal_bf16_bits(rng, (E, hidden), std=router_std),
            "sgate_bits": synth.normal_bf16_bits(rng, (hidden,), std=0.02),
            "shared": {"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)},
            "experts": [{"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)}
                        for _ in range(E)],
            "top_k": top_k}


def tokens(seed, m, hidden):
    return synth.normal_f16(np.random.default_rng([63, seed, m, hidden]), (m, hidden))


@pytest.fixture(scope="module")
def full():
    say("moe prefill workload E=256 hidden=2560 inter=512 top8 seed 0 (generating 256 experts)")
    d = synth.moe_workload(0)
    X = np.concatenate([d["x"][None], synth.moe_x_ring(0, 127)])
    return d, Layer(d), X


def test_prefill_workload_m128_bitwise_vs_decode(full):
    d, layer, X = full
    say("moe prefill m=128 vs 128 decodes")
    assert_bitwise(layer.prefill(X), layer.decodes(X), "m=128")


def test_prefill_workload_m128_oracle_every_row(full):
    d, layer, X = full
    say("moe prefill m=128 vs oracle (all 128 rows)")
    p = layer.prefill(X)
    check_oracle(d, X, p, range(128), what="m=128")


@pytest.mark.parametrize("m", [1, 2, 37, 127])
def test_prefill_workload_ragged_m_bitwise(full, m):
    d, layer, X = full
    say(f"moe prefill m={m} vs decodes")
    assert_bitwise(layer.prefill(X[:m]), layer.decodes(X[:m]), f"m={m}")


@pytest.mark.parametrize("E,hidden,inter,top_k,m", [
    (16, 512, 64, 3, 5), (16, 512, 64, 1, 9), (40, 1024, 128, 8, 128), (8, 512, 192, 8, 9),
    (300, 1536, 64, 5, 17), (1024, 512, 64, 8, 33), (9, 4096, 1024, 2, 3), (24, 2048, 576, 4, 20)])
def test_prefill_shapes(E, hidden, inter, top_k, m):
    say(f"moe prefill E={E} hidden={hidden} inter={inter} k={top_k} m={m}")
    d = small(0, E, hidden, inter, top_k)
    X = tokens(0, m, hidden)
    layer = Layer(d)
    p = layer.prefill(X)
    assert_bitwise(p, layer.decodes(X), f"E{E} m{m}")
    check_oracle(d, X, p, sorted({0, m // 2, m - 1}), what=f"E{E}")


@pytest.mark.parametrize("router_f32,boundary", [(True, False), (False, True), (True, True)])
def test_prefill_router_dtype_and_boundary(router_f32, boundary):
    say(f"moe prefill fp32 router={router_f32} fp16 boundary={boundary}")
    d = small(1, 32, 1024, 128, 4)
    X = tokens(1, 12, 1024)
    layer = Layer(d, router_f32=router_f32)
    p = layer.prefill(X, fp16_boundary=boundary)
    assert_bitwise(p, layer.decodes(X, fp16_boundary=boundary), "dtype/boundary")
    check_oracle(d, X, p, [0, 11], fp16_boundary=boundary, what="dtype/boundary")


def test_prefill_identical_tokens_share_one_route():
    """Every token the same: one expert set takes the whole chunk (a route list of m entries per
    selected expert) and every row equals the single decode."""
    say("moe prefill identical tokens")
    d = small(2, 64, 512, 64, 8)
    x = tokens(2, 1, 512)
    X = np.repeat(x, 128, axis=0)
    layer = Layer(d)
    out, ids, w = layer.prefill(X)
    one = layer.decodes(x)
    assert (ids == one[1][0]).all()
    assert (out.view(torch.int16) == one[0].view(torch.int16)[0]).all()
    assert torch.equal(w.view(torch.int32), one[2].view(torch.int32).expand(128, -1))


def test_prefill_ties_bitwise():
    """Router rows repeating with period 3: whole classes of experts tie, so the chunk's routing
    is decided by the lowest-index rule in every token."""
    say("moe prefill ties")
    d = small(3, 96, 512, 64, 8)
    d["router_bits"] = d["router_bits"][np.arange(96) % 3].copy()
    X = tokens(3, 16, 512)
    layer = Layer(d)
    p = layer.prefill(X)
    assert_bitwise(p, layer.decodes(X), "ties")
    check_oracle(d, X, p, [0, 15], what="ties")
