"""GPU: decodehp_moe_decode_noalloc (the library's fixed per-GPU scratch, no workspace) against
decodehp_moe_decode with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must agree bit for bit (fp16
output bits, ids, fp32 weight bits); the decode call itself is held to the fp64 oracle by
test_gpu_moe.py. Two calls in a row on the shared scratch, the second on a smaller layer, then
the first layer again: what a call leaves in the scratch never reaches the next one.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within_tol, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
hca = pytest.importorskip("hyper_connections_amd")


class Layer:
    def __init__(self, d):
        ex = d["experts"]
        self.d = d
        self.gate = hca.Int4Experts.from_logical([e["gate"] for e in ex])
        self.up = hca.Int4Experts.from_logical([e["up"] for e in ex])
        self.down = hca.Int4Experts.from_logical([e["down"] for e in ex])
        self.sg, self.su, self.sd = (hca.Int4Weight.from_logical(d["shared"][k].q, d["shared"][k].s_bits,
                                                                 d["shared"][k].b_bits) for k in ("gate", "up", "down"))
        self.router = hca.bf16_bits_to_tensor(d["router_bits"]).cuda()
        self.sgate = hca.bf16_bits_to_tensor(d["sgate_bits"]).cuda()
        self.k = d["top_k"]

    def args(self):
        return (self.router, self.sgate, self.gate, self.up, self.down, self.sg, self.su, self.sd, self.k)

    def both(self, x):
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        hidden = self.gate.cols
        out = torch.empty(hidden, dtype=torch.float16, device="cuda")
        ids = torch.empty(self.k, dtype=torch.int32, device="cuda")
        w = torch.empty(self.k, dtype=torch.float32, device="cuda")
        hca.moe_decode_noalloc(xd, *self.args(), out, ids, w)
        ref = hca.moe_decode(xd, *self.args())
        torch.cuda.synchronize()
        return (out.cpu(), ids.cpu(), w.cpu()), tuple(t.cpu() for t in ref)


def small_layer(seed=0, E=16, hidden=512, inter=64, top_k=3):
    rng = np.random.default_rng([91, seed])
    mk = lambda r, c: synth.int4_tensor(rng, r, c)
    return {"x": synth.normal_f16(rng, (hidden,)),
            "router_bits": synth.normal_bf16_bits(rng, (E, hidden), std=0.05),
            "sgate_bits": synth.normal_bf16_bits(rng, (hidden,), std=0.02),
            "shared": {"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)},
            "experts": [{"gate": mk(inter, hidden), "up": mk(inter, hidden), "down": mk(hidden, inter)}
                        for _ in range(E)],
            "top_k": top_k}


def assert_same(got, want, what):
    (o, i, w), (ro, ri, rw) = got, want
    assert torch.equal(i, ri), f"{what}: ids {i.tolist()} against {ri.tolist()}"
    assert torch.equal(o.view(torch.int16), ro.view(torch.int16)), f"{what}: output bits differ"
    assert torch.equal(w.view(torch.int32), rw.view(torch.int32)), f"{what}: weight bits differ"


def test_noalloc_matches_workspace_call_twice_then_smaller():
    say("moe noalloc: 256-expert top-8 layer, then a 16-expert top-3 layer, then the first again")
    big_d = synth.moe_workload(0)
    big, little = Layer(big_d), Layer(small_layer())
    a = big.both(big_d["x"])
    assert_same(*a, "256 experts, first call")
    b = little.both(little.d["x"])
    assert_same(*b, "16 experts, second call")
    ref = oracle.moe_decode(little.d["x"], little.d["router_bits"], little.d["sgate_bits"], little.d["shared"],
                            little.d["experts"], little.d["top_k"])
    assert b[0][1].tolist() == list(ref["ids"])
    assert_within_tol(b[0][0].float().numpy(), ref["out"], "16 experts vs oracle")
    x2 = synth.moe_x_ring(0, 1)[0]
    c = big.both(x2)
    assert_same(*c, "256 experts, third call")


def test_noalloc_rejects_a_layer_beyond_its_scratch():
    say("moe noalloc: layer larger than the fixed scratch")
    layer = Layer(small_layer(1, E=16, hidden=512, inter=1024, top_k=10))
    xd = torch.from_numpy(layer.d["x"]).cuda()
    out = torch.empty(512, dtype=torch.float16, device="cuda")
    ids = torch.empty(10, dtype=torch.int32, device="cuda")
    w = torch.empty(10, dtype=torch.float32, device="cuda")
    # (20 + 11 * 1024) * 4 bytes, rounded up to 256, + 9216 > 48 KiB
    with pytest.raises(hca.DecodeHPError) as e:
        hca.moe_decode_noalloc(xd, *layer.args(), out, ids, w)
    assert e.value.code == -4
