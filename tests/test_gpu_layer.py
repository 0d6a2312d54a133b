"""GPU: whole decoder layers (decodehp_decode_layers) and their captured graph.

  * the composed call against the same steps called one at a time through their own entry
    points: bit for bit (it is the same kernel sequence);
  * the graph against the eager call: bit for bit, on several tokens, replayed repeatedly with
    other eager GPU work and synchronisations between replays;
  * against the fp64 composition oracle (oracle.decode_layers): the residual and the mixer
    output within |d| <= 1e-3 + 1e-2 |oracle|.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within_tol, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
hca = pytest.importorskip("hyper_connections_amd")


def w4(t):
    return hca.Int4Weight.from_logical(t.q, t.s_bits, t.b_bits)


def block(b):
    return hca.HcBlock(hca.bf16_bits_to_tensor(b["gamma_bits"]).cuda(), w4(b["down"]), w4(b["up"]),
                       w4(b["inject"]) if b["inject"] is not None else None)


def dev_layers(d):
    out = []
    for L in d["layers"]:
        m = L["moe"]
        ex = m["experts"]
        out.append(hca.DecodeLayer(
            block(L["attn"]), w4(L["stub"]), block(L["mlp"]), hca.bf16_bits_to_tensor(m["router_bits"]).cuda(),
            hca.bf16_bits_to_tensor(m["sgate_bits"]).cuda(), hca.Int4Experts.from_logical([e["gate"] for e in ex]),
            hca.Int4Experts.from_logical([e["up"] for e in ex]), hca.Int4Experts.from_logical([e["down"] for e in ex]),
            w4(m["shared"]["gate"]), w4(m["shared"]["up"]), w4(m["shared"]["down"]), m["top_k"]))
    return out, block(d["mixer"])


def stepwise(x, C, H, layers, mixer):
    """The same layers through the individual entry points, one call per step."""
    hidden = x.repeat(C).contiguous()
    for L in layers:
        mixed, iw = hca.hc_read(hidden, L.attn_hc.hc_norm, C, H, L.attn_hc.down, L.attn_hc.up, L.attn_hc.inject)
        out = hca.dequant_gemv(L.sublayer, mixed)
        hca.hc_inject(hidden, out, iw, C, H)
        mixed, iw = hca.hc_read(hidden, L.mlp_hc.hc_norm, C, H, L.mlp_hc.down, L.mlp_hc.up, L.mlp_hc.inject)
        out, _, _ = hca.moe_decode(mixed, L.router, L.shared_gate_row, L.gate, L.up, L.down, L.shared_gate,
                                   L.shared_up, L.shared_down, L.top_k)
        hca.hc_inject(hidden, out, iw, C, H)
    mixed = hca.hc_read(hidden, mixer.hc_norm, C, H, mixer.down, mixer.up, None)
    mixed = mixed[0] if isinstance(mixed, tuple) else mixed
    return hidden, mixed


def bits(t):
    return t.view(torch.int16).cpu()


SMALL = dict(n_layers=2, c=4, h=512, r=64, n_experts=16, inter=64, top_k=4)


@pytest.fixture(scope="module")
def small():
    say("layers: 2 x (C=4 H=512 R=64 E=16 inter=64 k=4)")
    d = synth.decode_layer_workload(0, **SMALL)
    layers, mixer = dev_layers(d)
    return d, layers, mixer


def test_layers_equal_stepwise_calls(small):
    d, layers, mixer = small
    C, H = d["C"], d["H"]
    x = torch.from_numpy(d["x"]).cuda()
    h1, m1 = hca.decode_layers(x, C, H, layers, mixer)
    h2, m2 = stepwise(x, C, H, layers, mixer)
    torch.cuda.synchronize()
    assert torch.equal(bits(h1), bits(h2)) and torch.equal(bits(m1), bits(m2))


def test_layers_vs_oracle_small(small):
    d, layers, mixer = small
    C, H = d["C"], d["H"]
    x = torch.from_numpy(d["x"]).cuda()
    h, m = hca.decode_layers(x, C, H, layers, mixer)
    torch.cuda.synchronize()
    ref = oracle.decode_layers(d["x"], d["layers"], d["mixer"], C, H)
    assert_within_tol(h.float().cpu().numpy(), ref["hidden"], "hidden")
    assert_within_tol(m.float().cpu().numpy(), ref["mixed"], "mixed")


def test_graph_replays_equal_eager(small):
    d, layers, mixer = small
    C, H = d["C"], d["H"]
    xs = synth.normal_f16(np.random.default_rng(91), (4, H))
    xg = torch.empty(H, dtype=torch.float16, device="cuda")
    hg = torch.empty(C * H, dtype=torch.float16, device="cuda")
    mg = torch.empty(H, dtype=torch.float16, device="cuda")
    xg.copy_(torch.from_numpy(xs[0]))
    g = hca.LayerGraph(xg, C, H, layers, mixer, hg, mg)
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(4):
            say(f"graph replay {rep} token {i}")
            xg.copy_(torch.from_numpy(xs[i]))
            g.launch()
            torch.cuda.synchronize()
            he, me = hca.decode_layers(torch.from_numpy(xs[i]).cuda(), C, H, layers, mixer)   # eager, in between
            torch.cuda.synchronize()
            assert torch.equal(bits(hg), bits(he)), (rep, i)
            assert torch.equal(bits(mg), bits(me)), (rep, i)


def test_zero_layers_is_replicate_and_mixer(small):
    d, layers, mixer = small
    C, H = d["C"], d["H"]
    x = torch.from_numpy(d["x"]).cuda()
    h, m = hca.decode_layers(x, C, H, [], mixer)
    torch.cuda.synchronize()
    assert torch.equal(bits(h), bits(x.repeat(C)))
    ref = oracle.decode_layers(d["x"], [], d["mixer"], C, H)
    assert_within_tol(m.float().cpu().numpy(), ref["mixed"], "mixer only")


def test_layer_full_size_vs_oracle():
    say("layers: 1 x (C=4 H=2560 R=320 E=256 inter=512 k=8), generating 256 experts")
    d = synth.decode_layer_workload(0, n_layers=1)
    layers, mixer = dev_layers(d)
    C, H = d["C"], d["H"]
    x = torch.from_numpy(d["x"]).cuda()
    h, m = hca.decode_layers(x, C, H, layers, mixer)
    torch.cuda.synchronize()
    ref = oracle.decode_layers(d["x"], d["layers"], d["mixer"], C, H)
    assert_within_tol(h.float().cpu().numpy(), ref["hidden"], "hidden")
    assert_within_tol(m.float().cpu().numpy(), ref["mixed"], "mixed")
