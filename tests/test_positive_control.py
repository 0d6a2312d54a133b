"""The tolerance bar can see precision loss (CPU only).

"src/real_forward.rs", field batched_gemv_prefill: the pages prove their parity fixture
can detect a non-exact kernel with a positive control that differs on a large share of
outputs. Here the control is planted on the CPU: the batched workload computed with both
GEMM operands rounded to bfloat16 must FAIL the |d| <= 1e-3 + 1e-2|oracle| bar on a
visible share of outputs, while fp16 operands (what the matrix-core arm uses) pass.
"""
import numpy as np

import oracle
import synth
from helpers import tol_violations


def _bf16(a):
    return oracle.bf16_bits_to_f64(synth.to_bf16_bits(a))


def test_bf16_operands_fail_and_fp16_operands_pass():
    d = synth.prefill_workload(0)
    cols = slice(0, 512)                       # a column sample keeps this test to a second
    w = d["w"]
    W = oracle.dequant(w.q[cols], w.s_bits[cols], w.b_bits[cols])
    X = d["x"].astype(np.float64)
    ref = X @ W.T
    fp16 = X @ W.astype(np.float16).astype(np.float64).T
    bf16 = _bf16(X) @ _bf16(W).T
    n16, _ = tol_violations(fp16, ref)
    nbf, _ = tol_violations(bf16, ref)
    assert n16 == 0
    assert nbf > 0.02 * ref.size, nbf
    # the dequantized weights of this workload are exact in fp16 (bias = -8 * scale)
    assert np.array_equal(W.astype(np.float16).astype(np.float64), W)
