"""GPU parity: decodehp_hc_read / decodehp_hc_inject against the fp64 oracle.

Bar: |gpu - oracle| <= 1e-3 + 1e-2 |oracle| elementwise (mixed, inject_w, hidden).
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


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_read(raw, gamma_bits, down, up, inject, C, H):
    mixed, iw = hca.hc_read(to_dev(raw), hca.bf16_bits_to_tensor(gamma_bits).cuda(), C, H, dev_int4(down),
                            dev_int4(up), dev_int4(inject) if inject is not None else None)
    torch.cuda.synchronize()
    return mixed.float().cpu().numpy(), (iw.cpu().numpy() if iw is not None else None)


def test_hc_workload_c4_h2560():
    say("hc read+inject C=4 H=2560 R=320 seed 0")
    d = synth.hc_workload(0)
    C, H = d["C"], d["H"]
    mixed, iw = gpu_read(d["raw"], d["gamma_bits"], d["down"], d["up"], d["inject"], C, H)
    ref = oracle.hc_read(d["raw"], d["gamma_bits"], d["down"], d["up"], d["inject"], C, H)
    assert_within_tol(mixed, ref["mixed"], "mixed")
    assert_within_tol(iw, ref["inject_w"], "inject_w")
    # inject with the workload's own sublayer output and inject weights
    wide = to_dev(d["raw"])
    hca.hc_inject(wide, to_dev(d["out"]), to_dev(d["iw"]), C, H)
    torch.cuda.synchronize()
    hidden_ref = oracle.hc_inject(d["raw"], d["out"], d["iw"], C, H)
    assert_within_tol(wide.float().cpu().numpy(), hidden_ref, "hidden")


@pytest.mark.parametrize("C,H,R", [(1, 2048, 64), (2, 1024, 128), (4, 512, 64), (8, 256, 192),
                                   (16, 128, 64), (2, 4096, 320), (4, 2560, 1024), (1, 8192, 320)])
def test_hc_read_shapes(C, H, R):
    say(f"hc read C={C} H={H} R={R}")
    rng = np.random.default_rng([51, C, H, R])
    raw = synth.normal_f16(rng, (C * H,))
    gam = synth.normal_bf16_bits(rng, (C * H,), mean=1.0, std=0.02)
    down, up, inj = synth.int4_tensor(rng, R, C * H), synth.int4_tensor(rng, C * H, R), synth.int4_tensor(rng, C, C * H)
    mixed, iw = gpu_read(raw, gam, down, up, inj, C, H)
    ref = oracle.hc_read(raw, gam, down, up, inj, C, H)
    assert_within_tol(mixed, ref["mixed"], f"mixed C={C}")
    assert_within_tol(iw, ref["inject_w"], f"inject_w C={C}")


def test_hc_final_mixer_without_inject():
    say("hc final mixer (no inject)")
    d = synth.hc_workload(3)
    mixed, iw = gpu_read(d["raw"], d["gamma_bits"], d["down"], d["up"], None, d["C"], d["H"])
    ref = oracle.hc_read(d["raw"], d["gamma_bits"], d["down"], d["up"], None, d["C"], d["H"])
    assert iw is None
    assert_within_tol(mixed, ref["mixed"], "final mixer")


def test_hc_zero_up_gives_half_mean_normed():
    say("hc zero up")
    d = synth.hc_workload(4)
    C, H, R = d["C"], d["H"], d["R"]
    up0 = synth.Int4Tensor(np.full((C * H, R), 8, np.uint8), d["up"].s_bits, d["up"].b_bits)
    mixed, _ = gpu_read(d["raw"], d["gamma_bits"], d["down"], up0, d["inject"], C, H)
    n = oracle.grouped_rmsnorm(d["raw"], d["gamma_bits"], C, H).reshape(C, H)
    assert_within_tol(mixed, 0.5 * n.mean(axis=0), "0.5 * mean normed")


def test_hc_inject_c1_is_plain_residual_add():
    say("hc inject C=1 iw=1")
    rng = np.random.default_rng(52)
    raw = synth.normal_f16(rng, (2560,))
    out = synth.normal_f16(rng, (2560,))
    wide = to_dev(raw)
    hca.hc_inject(wide, to_dev(out), torch.ones(1, device="cuda"), 1, 2560)
    torch.cuda.synchronize()
    got = wide.cpu().numpy()
    assert np.array_equal(got, (raw.astype(np.float32) + out.astype(np.float32)).astype(np.float16))
    assert_within_tol(got, oracle.hc_inject(raw, out, [1.0], 1, 2560), "C=1 add")


def test_hc_inject_zero_weights_leave_raw_bitwise():
    say("hc inject iw=0")
    rng = np.random.default_rng(53)
    raw = synth.normal_f16(rng, (4 * 2560,))
    out = synth.normal_f16(rng, (2560,))
    wide = to_dev(raw)
    hca.hc_inject(wide, to_dev(out), torch.zeros(4, device="cuda"), 4, 2560)
    torch.cuda.synchronize()
    assert np.array_equal(wide.cpu().numpy(), raw)


@pytest.mark.parametrize("C,H", [(3, 8), (16, 64), (4, 2560), (1, 8)])
def test_hc_inject_shapes(C, H):
    say(f"hc inject C={C} H={H}")
    rng = np.random.default_rng([54, C, H])
    raw = synth.normal_f16(rng, (C * H,))
    out = synth.normal_f16(rng, (H,))
    iw = rng.uniform(0, 2, size=C).astype(np.float32)
    wide = to_dev(raw)
    hca.hc_inject(wide, to_dev(out), to_dev(iw), C, H)
    torch.cuda.synchronize()
    assert_within_tol(wide.float().cpu().numpy(), oracle.hc_inject(raw, out, iw, C, H), "inject")


def test_hc_read_deterministic_and_guarded():
    say("hc determinism + guard")
    d = synth.hc_workload(5)
    C, H = d["C"], d["H"]
    args = (to_dev(d["raw"]), hca.bf16_bits_to_tensor(d["gamma_bits"]).cuda(), C, H, dev_int4(d["down"]),
            dev_int4(d["up"]), dev_int4(d["inject"]))
    buf = torch.full((H + 256,), -7.0, dtype=torch.float16, device="cuda")
    wbuf = torch.full((C + 8,), -7.0, dtype=torch.float32, device="cuda")
    m1, w1 = hca.hc_read(*args, mixed=buf[128:128 + H], inject_w=wbuf[4:4 + C])
    a, b = m1.clone(), w1.clone()
    hca.hc_read(*args, mixed=buf[128:128 + H], inject_w=wbuf[4:4 + C])
    torch.cuda.synchronize()
    assert torch.equal(a, buf[128:128 + H]) and torch.equal(b, wbuf[4:4 + C])
    assert torch.all(buf[:128] == -7.0) and torch.all(buf[128 + H:] == -7.0)
    assert torch.all(wbuf[:4] == -7.0) and torch.all(wbuf[4 + C:] == -7.0)


@pytest.mark.parametrize("C,H,R,inject", [(4, 2560, 320, True), (4, 2560, 320, False), (2, 1024, 128, True),
                                          (16, 128, 64, True), (1, 8192, 320, True)])
def test_hc_inject_read_is_inject_then_read_bitwise(C, H, R, inject):
    """decodehp_hc_inject_read (the inject formed inside the read's first kernel) against
    decodehp_hc_inject followed by decodehp_hc_read: the same bits for the new residual, mixed and
    the new inject weights; prev is left unchanged; and the oracle's inject then read."""
    say(f"hc inject+read C={C} H={H} R={R} inject={inject}")
    rng = np.random.default_rng([52, C, H, R])
    blk = synth.hc_block(rng, C, H, R, inject=inject)
    prev = synth.normal_f16(rng, (C * H,))
    out = synth.normal_f16(rng, (H,))
    iw = rng.uniform(0.0, 2.0, size=C).astype(np.float32)
    gamma = hca.bf16_bits_to_tensor(blk["gamma_bits"]).cuda()
    down, up = dev_int4(blk["down"]), dev_int4(blk["up"])
    inj = dev_int4(blk["inject"]) if inject else None
    prev_d, out_d, iw_d = to_dev(prev), to_dev(out), to_dev(iw)
    hidden, mixed, iw_next = hca.hc_inject_read(prev_d, out_d, iw_d, gamma, C, H, down, up, inj)
    wide = prev_d.clone()
    hca.hc_inject(wide, out_d, iw_d, C, H)
    mixed2, iw2 = hca.hc_read(wide, gamma, C, H, down, up, inj)
    torch.cuda.synchronize()
    assert torch.equal(prev_d.cpu(), torch.from_numpy(prev))
    assert torch.equal(hidden.view(torch.int16).cpu(), wide.view(torch.int16).cpu())
    assert torch.equal(mixed.view(torch.int16).cpu(), mixed2.view(torch.int16).cpu())
    if inject:
        assert torch.equal(iw_next.view(torch.int32).cpu(), iw2.view(torch.int32).cpu())
    hid_ref = oracle.hc_inject(prev, out, iw, C, H)
    assert_within_tol(hidden.float().cpu().numpy(), hid_ref, "hidden")
    ref = oracle.hc_read(hidden.cpu().numpy(), blk["gamma_bits"], blk["down"], blk["up"], blk["inject"] if inject else None,
                         C, H)
    assert_within_tol(mixed.float().cpu().numpy(), ref["mixed"], "mixed after inject")
    if inject:
        assert_within_tol(iw_next.cpu().numpy(), ref["inject_w"], "inject_w after inject")
