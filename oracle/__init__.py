"""CPU oracle for the decode hot path -- TEST INFRASTRUCTURE, not product code.

Plain, slow, obviously correct fp64 NumPy implementations of what the GPU library
computes. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package; the product path (``hyper_connections_amd``) never does and
shares no code with it.

Sources (the turbospark-runtime 0.3.0 docs.rs pages):
  * "src/families/qwen4/mod.rs" -- module doc, sections "The decoder layer, as
    pseudocode", "THE INJECTION TRAP", "Hyper-connections", "MoE"; constant RMS_EPS.
  * "src/families/qwen4/hc.rs" -- doc of encode_hyper_connection and its body
    (grouped RMS norm, down GEMV, 1/C scale, SiLU, up GEMV, sigmoid, hc_mix, inject
    GEMV, 1/C, sigmoid, x2).
  * "src/families/qwen/state.rs" -- struct RealQwenState fields router_ones,
    per_expert_ones, router_logits_f32, moe_x, h1, h2, shared_gate_logit.
  * "src/families/qwen4/mod.rs", module doc, "The decoder layer, as pseudocode" -- the
    whole-layer composition (oracle/layer.py).
  * "src/real_forward.rs" -- module doc (INT4-affine resident weights bound as
    weights/scales/biases; MoE phase-1 gate/up + activation and phase-2 down + k-way
    reduce; host top-k + softmax) and field batched_gemv_prefill.

Every input is decoded exactly to float64 (fp16 and bf16 are subsets of float64) and
every intermediate stays float64. Outputs are returned unrounded; callers round to
the output dtype when they compare.

Parity status per function is listed in the module docstrings. Each function here is
pinned by the not-gpu tests in tests/test_oracle_*.py against closed forms,
invariants and exact brute force; see the test files for the pin list.
"""
from .int4 import bf16_bits_to_f64, dequant                        # noqa: F401
from .gemv import dequant_gemv, argmax_lowest                      # noqa: F401
from .moe import (router_logits, select_topk, softmax_selected,   # noqa: F401
                  expert_act, expert_down, moe_decode, moe_prefill)
from .hc import grouped_rmsnorm, hc_read, hc_inject, hc_read_batched, hc_inject_batched  # noqa: F401
from .layer import decode_layers                                    # noqa: F401
