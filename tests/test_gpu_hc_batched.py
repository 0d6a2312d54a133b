"""GPU parity: decodehp_hc_read_batched / decodehp_hc_inject_batched (a chunk of m tokens)
against the fp64 oracle, row by row.

Bar: mixed and inject_w within |d| <= 1e-3 + 1e-2 |oracle| elementwise; the inject's fp16 rows
within the same bar of the fp64 inject of the same fp16 inputs. The batched read is not bit for
bit the per-token read (its projections run as matrix-core GEMMs over fp16 operands).
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


def run(blk, rows, C, H, inject=True):
    raw = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
    gamma = hca.bf16_bits_to_tensor(blk["gamma_bits"]).cuda()
    mixed, iw = hca.hc_read_batched(raw, gamma, C, H, w4(blk["down"]), w4(blk["up"]),
                                    w4(blk["inject"]) if inject else None)
    torch.cuda.synchronize()
    return mixed.float().cpu().numpy(), (iw.cpu().numpy() if iw is not None else None)


def check_rows(blk, rows, C, H, mixed, iw, which, inject=True, what="hcb"):
    for t in which:
        ref = oracle.hc_read(rows[t], blk["gamma_bits"], blk["down"], blk["up"], blk["inject"] if inject else None,
                             C, H)
        assert_within_tol(mixed[t], ref["mixed"], f"{what} row {t} mixed")
        if inject:
            assert_within_tol(iw[t], ref["inject_w"], f"{what} row {t} inject_w")


@pytest.fixture(scope="module")
def workload():
    say("hc batched workload C=4 H=2560 R=320 m=128")
    h = synth.hc_workload(0)
    rng = np.random.default_rng([64, 0])
    rows = np.concatenate([h["raw"][None], synth.normal_f16(rng, (127, 4 * 2560))])
    blk = {"gamma_bits": h["gamma_bits"], "down": h["down"], "up": h["up"], "inject": h["inject"]}
    return blk, rows


@pytest.mark.parametrize("m", [1, 7, 128])
def test_hc_read_batched_workload(workload, m):
    blk, rows = workload
    say(f"hc batched m={m}")
    mixed, iw = run(blk, rows[:m], 4, 2560)
    check_rows(blk, rows, 4, 2560, mixed, iw, range(m), what=f"m={m}")


def test_hc_read_batched_final_mixer(workload):
    blk, rows = workload
    say("hc batched mixer m=9")
    mixed, iw = run(blk, rows[:9], 4, 2560, inject=False)
    assert iw is None
    check_rows(blk, rows, 4, 2560, mixed, iw, [0, 8], inject=False, what="mixer")


@pytest.mark.parametrize("C,H,R,m", [(1, 2048, 64, 3), (2, 1024, 128, 65), (16, 128, 64, 5), (8, 4096, 1024, 2)])
def test_hc_read_batched_shapes(C, H, R, m):
    say(f"hc batched C={C} H={H} R={R} m={m}")
    rng = np.random.default_rng([65, C, H, R, m])
    blk = synth.hc_block(rng, C, H, R)
    rows = synth.normal_f16(rng, (m, C * H))
    mixed, iw = run(blk, rows, C, H)
    check_rows(blk, rows, C, H, mixed, iw, sorted({0, m - 1}), what=f"C{C}")


def test_hc_inject_batched_rows(workload):
    blk, rows = workload
    say("hc inject batched m=33")
    m, C, H = 33, 4, 2560
    rng = np.random.default_rng(66)
    out = synth.normal_f16(rng, (m, H))
    w = rng.uniform(0.0, 2.0, size=(m, C)).astype(np.float32)
    wide = torch.from_numpy(np.ascontiguousarray(rows[:m])).cuda()
    hca.hc_inject_batched(wide, torch.from_numpy(out).cuda(), torch.from_numpy(w).cuda(), C, H)
    torch.cuda.synchronize()
    ref = oracle.hc_inject_batched(rows[:m].astype(np.float64), out.astype(np.float64), w.astype(np.float64), C, H)
    assert_within_tol(wide.float().cpu().numpy(), ref, "inject rows")


@pytest.mark.parametrize("m,inject", [(33, True), (100, True), (65, False)])
def test_hc_read_batched_every_row_past_32(workload, m, inject):
    # More than 32 tokens at C = 4 take the up projection with the stream mix in its epilogue
    # (64-row tiles, the last one ragged): every row against the oracle.
    blk, rows = workload
    say(f"hc batched every row m={m} inject={inject}")
    mixed, iw = run(blk, rows[:m], 4, 2560, inject=inject)
    check_rows(blk, rows, 4, 2560, mixed, iw, list(range(m)), inject=inject, what=f"all m={m}")
