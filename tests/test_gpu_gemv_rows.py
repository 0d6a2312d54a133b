"""GPU: the multi-row decodehp_dequant_gemv (2 <= m <= 16) against m single-row calls.

"src/real_forward.rs", field batched_gemv_prefill: the batched GEMV and the per-row GEMV agree
bit for bit. Bar: every row's fp32 logits bit for bit equal to the m = 1 call on that row alone,
its argmax equal, and the rows within |d| <= 1e-3 + 1e-2 |oracle| of the fp64 oracle. Shapes
cover ragged row counts (not a multiple of the 256-row block), K with a partial last segment of
16 chunks (K % 512 != 0, where the m = 1 call takes its LDS kernel), activation rows in two
passes (m > 8), and biases other than -8 * scale. Row counts that are multiples of 16 with an even
number of groups (at most 48) take each tile's scales and biases as one coalesced block; the
others take them per chunk.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within_tol, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
hca = pytest.importorskip("hyper_connections_amd")


def dev(t):
    return hca.Int4Weight.from_logical(t.q, t.s_bits, t.b_bits)


def rows_and_singles(w, X):
    xd = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    y, am = hca.dequant_gemv(w, xd, out_dtype=torch.float32, argmax=True)
    singles = [hca.dequant_gemv(w, xd[r], out_dtype=torch.float32, argmax=True) for r in range(X.shape[0])]
    torch.cuda.synchronize()
    ys = torch.stack([s[0].reshape(-1) for s in singles]).cpu()
    ams = torch.cat([s[1] for s in singles]).cpu()
    return y.cpu(), am.cpu(), ys, ams


def assert_bitwise(y, am, ys, ams, what):
    bad = (y.view(torch.int32) != ys.view(torch.int32)).nonzero()
    assert bad.numel() == 0, f"{what}: {bad.shape[0]} outputs differ from the single-row calls, first {bad[:4].tolist()}"
    assert torch.equal(am, ams), f"{what}: argmax {am.tolist()} against {ams.tolist()}"


def general_bias(rng, t):
    """The same codes and scales with biases other than -8 * scale (bf16 of s * U(-12, -4))."""
    s = synth.bf16_bits_to_f32(t.s_bits).astype(np.float64)
    b = synth.to_bf16_bits(-s * rng.uniform(4.0, 12.0, size=s.shape))
    return synth.Int4Tensor(t.q, t.s_bits, b)


@pytest.mark.parametrize("m", [2, 3, 5, 8, 9, 16])
def test_rows_bitwise_equal_single_row_calls(m):
    say(f"gemv rows m={m} n=5000 k=2560")
    rng = np.random.default_rng([91, m])
    t = synth.int4_tensor(rng, 5000, 2560)
    X = synth.normal_f16(rng, (m, 2560))
    y, am, ys, ams = rows_and_singles(dev(t), X)
    assert_bitwise(y, am, ys, ams, f"m={m}")
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert_within_tol(y.numpy(), ref, f"rows m={m}")
    assert am.numpy().tolist() == oracle.argmax_lowest(ref).tolist()


@pytest.mark.parametrize("n,k", [(300, 64), (1001, 640), (513, 1216), (2000, 4096), (257, 16384), (40, 7744)])
def test_rows_bitwise_shapes(n, k):
    say(f"gemv rows m=4 n={n} k={k}")
    rng = np.random.default_rng([92, n, k])
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (4, k))
    y, am, ys, ams = rows_and_singles(dev(t), X)
    assert_bitwise(y, am, ys, ams, f"n={n} k={k}")
    assert_within_tol(y.numpy(), oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X), f"rows n={n} k={k}")


@pytest.mark.parametrize("n,k,m", [(4096, 2560, 8), (1024, 640, 4), (512, 1152, 6), (2048, 1536, 12),
                                   (256, 128, 3), (64, 3072, 4)])
def test_rows_bitwise_tile_block(n, k, m):
    """Whole tiles, G even: the tile-block path, with whole and partial last super-steps, one and
    two groups of activation rows, and two passes; the smallest block (K = 128, a super-step
    mostly padding) and the largest (K = 3072, 64 G = 3072 bytes, which fits the LDS at m <= 4)."""
    say(f"gemv rows tile block m={m} n={n} k={k}")
    rng = np.random.default_rng([95, n, k, m])
    t = general_bias(rng, synth.int4_tensor(rng, n, k))
    X = synth.normal_f16(rng, (m, k))
    y, am, ys, ams = rows_and_singles(dev(t), X)
    assert_bitwise(y, am, ys, ams, f"tile block n={n} k={k} m={m}")
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert_within_tol(y.numpy(), ref, f"rows tile block n={n} k={k} m={m}")
    assert am.numpy().tolist() == oracle.argmax_lowest(ref).tolist()


def test_rows_bitwise_general_biases():
    say("gemv rows m=6, biases other than -8 * scale")
    rng = np.random.default_rng(93)
    t = general_bias(rng, synth.int4_tensor(rng, 3000, 2560))
    X = synth.normal_f16(rng, (6, 2560))
    y, am, ys, ams = rows_and_singles(dev(t), X)
    assert_bitwise(y, am, ys, ams, "general biases")
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert_within_tol(y.numpy(), ref, "rows, general biases")
    assert am.numpy().tolist() == oracle.argmax_lowest(ref).tolist()


def test_rows_fp16_output_is_rounded_fp32():
    say("gemv rows fp16 vs fp32 outputs")
    rng = np.random.default_rng(94)
    t = synth.int4_tensor(rng, 700, 1024)
    xd = torch.from_numpy(synth.normal_f16(rng, (5, 1024))).cuda()
    w = dev(t)
    y32 = hca.dequant_gemv(w, xd, out_dtype=torch.float32)
    y16 = hca.dequant_gemv(w, xd)
    torch.cuda.synchronize()
    assert torch.equal(y16.cpu(), y32.cpu().half())


def test_lmhead_m8_bitwise_equal_eight_m1_calls():
    say("lm head 151936x2560: M=8 against eight M=1 calls")
    d = synth.lmhead_workload(0, m=8)
    y, am, ys, ams = rows_and_singles(dev(d["w"]), d["x"])
    assert_bitwise(y, am, ys, ams, "lm head M=8")
    ref = oracle.dequant_gemv(d["w"].q, d["w"].s_bits, d["w"].b_bits, d["x"])
    assert_within_tol(y.numpy(), ref, "lm head M=8 rows")
    assert am.numpy().tolist() == oracle.argmax_lowest(ref).tolist()


def test_matrix_core_arm_general_biases_within_bar_or_reported():
    """The matrix-core arm rounds every dequantized weight to fp16: exact for bias = -8 * scale,
    not in general. Its results with general biases are checked against the oracle at a looser
    bar that accounts for half an fp16 ulp per weight (sum of |x| times the largest weight's
    half-ulp), and the count of outputs past the plain bar is printed."""
    say("gemv matrix-core arm, general biases")
    rng = np.random.default_rng(95)
    t = general_bias(rng, synth.int4_tensor(rng, 3000, 2560))
    X = synth.normal_f16(rng, (8, 2560))
    y, am = hca.dequant_gemv(dev(t), torch.from_numpy(X).cuda(), out_dtype=torch.float32, argmax=True,
                             matrix_cores=True)
    torch.cuda.synchronize()
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    W = oracle.dequant(t.q, t.s_bits, t.b_bits)
    half_ulp = np.spacing(np.abs(W).astype(np.float16)).astype(np.float64) / 2      # fp16 spacing
    allowance = np.abs(X.astype(np.float64)) @ half_ulp.T
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-3 + 1e-2 * np.abs(ref) + allowance)
    plain = int(np.sum(err > 1e-3 + 1e-2 * np.abs(ref)))
    print(f"matrix-core arm, general biases: {plain} of {ref.size} outputs past the plain bar")
