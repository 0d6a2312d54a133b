"""GPU parity: decodehp_dequant_gemm_batched (m <= 128, matrix cores) and the multi-row
decodehp_dequant_gemv (2 <= m <= 16, with argmax) -- both its default arm, bit-equal to single-row
calls (tests/test_gpu_gemv_rows.py holds that), and its matrix-core arm (decodehp_dequant_gemv_mc)
-- against the fp64 oracle.

Bar: |gpu - oracle| <= 1e-3 + 1e-2 |oracle| elementwise; argmax bit-exact.
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


def batched(t, X):
    y = hca.dequant_gemm_batched(dev(t), torch.from_numpy(np.ascontiguousarray(X)).cuda())
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def test_prefill_workload_m128():
    say("batched M=128 N=8192 K=2560 seed 0")
    d = synth.prefill_workload(0)
    y = batched(d["w"], d["x"])
    ref = oracle.dequant_gemv(d["w"].q, d["w"].s_bits, d["w"].b_bits, d["x"])
    assert_within_tol(y, ref, "prefill M=128")


@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (2, 48, 128), (5, 80, 320), (31, 64, 2560), (32, 1024, 2560),
                                   (33, 64, 192), (64, 1040, 512), (100, 256, 2560), (128, 16, 64),
                                   (128, 4096, 4096), (7, 160, 10240), (3, 48, 32768), (65, 80, 16384),
                                   (127, 208, 1216)])
def test_batched_shapes(m, n, k):
    say(f"batched m={m} n={n} k={k}")
    rng = np.random.default_rng([71, m, n, k])
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (m, k))
    assert_within_tol(batched(t, X), oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X), f"batched {m}x{n}x{k}")


def test_batched_rows_independent_of_block():
    # the same activation row computed in different M tiles gives the same bits
    say("batched row independence")
    rng = np.random.default_rng(72)
    t = synth.int4_tensor(rng, 256, 1024)
    X = synth.normal_f16(rng, (128, 1024))
    X[100] = X[3]
    y = batched(t, X)
    assert np.array_equal(y[100], y[3])


@pytest.mark.parametrize("mc", [False, True])
@pytest.mark.parametrize("m", [2, 3, 8, 16])
def test_gemv_multirow_with_argmax(m, mc):
    say(f"gemv multi-row m={m} matrix_cores={mc}")
    rng = np.random.default_rng([73, m])
    n, k = 20000, 2560
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (m, k))
    y, am = hca.dequant_gemv(dev(t), torch.from_numpy(X).cuda(), out_dtype=torch.float32, argmax=True,
                             matrix_cores=mc)
    torch.cuda.synchronize()
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert_within_tol(y.cpu().numpy(), ref, f"gemv m={m}")
    assert am.cpu().numpy().tolist() == oracle.argmax_lowest(ref).tolist()
    y16 = hca.dequant_gemv(dev(t), torch.from_numpy(X).cuda(), matrix_cores=mc)
    torch.cuda.synchronize()
    assert torch.equal(y16.cpu(), y.cpu().half())


@pytest.mark.parametrize("mc", [False, True])
def test_lmhead_m8_full_vocab_with_argmax(mc):
    say(f"lm head 151936x2560 M=8 fp32 + argmax, matrix_cores={mc}")
    d = synth.lmhead_workload(0, m=8)
    y, am = hca.dequant_gemv(dev(d["w"]), torch.from_numpy(d["x"]).cuda(), out_dtype=torch.float32, argmax=True,
                             matrix_cores=mc)
    torch.cuda.synchronize()
    ref = oracle.dequant_gemv(d["w"].q, d["w"].s_bits, d["w"].b_bits, d["x"])
    assert_within_tol(y.cpu().numpy(), ref, "lm head M=8")
    assert am.cpu().numpy().tolist() == oracle.argmax_lowest(ref).tolist()
    gaps = [float(np.diff(np.sort(r)[-2:])[0]) for r in ref]
    print("top-1/top-2 gaps", ", ".join(f"{g:.3f}" for g in gaps))


@pytest.mark.parametrize("mc", [False, True])
def test_multirow_argmax_tie_lowest_index(mc):
    say(f"gemv multi-row argmax tie, matrix_cores={mc}")
    rng = np.random.default_rng(74)
    n, k, m = 30000, 2560, 4
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (m, k))
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    a = int(oracle.argmax_lowest(ref[2]))
    b = (a + 12345) % n
    for arr in (t.q, t.s_bits, t.b_bits):
        arr[b] = arr[a]
    y, am = hca.dequant_gemv(dev(t), torch.from_numpy(X).cuda(), out_dtype=torch.float32, argmax=True,
                             matrix_cores=mc)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert y[2, a] == y[2, b]
    assert int(am.cpu()[2]) == min(a, b)


@pytest.mark.parametrize("mc", [False, True])
def test_multirow_argmax_repeated_calls(mc):
    say(f"multi-row argmax repeated calls, matrix_cores={mc}")
    rng = np.random.default_rng(75)
    n, k, m = 9000, 1024, 5
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (m, k))
    ref = oracle.argmax_lowest(oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)).tolist()
    w = dev(t)
    xd = torch.from_numpy(X).cuda()
    outs = [hca.dequant_gemv(w, xd, out_dtype=torch.float32, argmax=True, matrix_cores=mc)[1] for _ in range(10)]
    torch.cuda.synchronize()
    assert all(o.cpu().numpy().tolist() == ref for o in outs)


@pytest.mark.parametrize("mc", [False, True])
@pytest.mark.parametrize("m,n,k", [(2, 33, 128), (5, 17, 640), (9, 4099, 1280), (16, 1000, 2560), (3, 1, 2560),
                                   (12, 16, 384), (2, 70001, 2560)])
def test_gemv_multirow_ragged_tiles(m, n, k, mc):
    # tiles of 16 weight rows with a ragged last tile; K a multiple of 128 up to 2560
    say(f"gemv multi-row ragged m={m} n={n} k={k} matrix_cores={mc}")
    rng = np.random.default_rng([76, m, n, k])
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (m, k))
    y, am = hca.dequant_gemv(dev(t), torch.from_numpy(X).cuda(), out_dtype=torch.float32, argmax=True,
                             matrix_cores=mc)
    torch.cuda.synchronize()
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert_within_tol(y.cpu().numpy(), ref, f"gemv m={m} n={n} k={k}")
    assert am.cpu().numpy().tolist() == oracle.argmax_lowest(ref).tolist()


def test_gemv_multirow_scales_at_odd_halfword():
    # scale/bias arrays that are only 2-byte aligned take the other matrix-core arm; same results
    say("gemv multi-row, scales 2-byte aligned")
    rng = np.random.default_rng(77)
    m, n, k = 6, 3000, 2560
    t = synth.int4_tensor(rng, n, k)
    X = synth.normal_f16(rng, (m, k))
    w = dev(t)
    g = k // 64
    s_store = torch.zeros(n * g + 1, dtype=torch.int16, device="cuda")
    b_store = torch.zeros(n * g + 1, dtype=torch.int16, device="cuda")
    s_store[1:] = w.scales.reshape(-1)
    b_store[1:] = w.biases.reshape(-1)
    odd = hca.Int4Weight(w.codes, s_store[1:].view(n, g), b_store[1:].view(n, g), n, k)
    xd = torch.from_numpy(X).cuda()
    y_odd, am_odd = hca.dequant_gemv(odd, xd, out_dtype=torch.float32, argmax=True, matrix_cores=True)
    torch.cuda.synchronize()
    ref = oracle.dequant_gemv(t.q, t.s_bits, t.b_bits, X)
    assert_within_tol(y_odd.cpu().numpy(), ref, "gemv m=6 odd-halfword scales")
    assert am_odd.cpu().numpy().tolist() == oracle.argmax_lowest(ref).tolist()
