#!/usr/bin/env python3
"""Benchmark of the MI355X decode hot path (libdecodehp) on one GPU.

One step = one pass of every hot-path call over one batch of seeded synthetic inputs:

  gemv      INT4 dequant GEMV, M=1, 2560 x 2560, fp16 out
  hc        hyper-connection read (C=4, H=2560, R=320, with inject gate) + inject add
  moe       routed MoE decode, 256 resident experts, top-8, gated shared expert
  prefill   batched projection, M=128, N=8192, K=2560 (matrix cores), fp16 out
  lmhead1   LM head, M=1, 151936 x 2560, fp32 logits + argmax
  lmhead8   LM head, M=8, same shape, fp32 logits + argmax (the default multi-row arm, whose
            logits are bitwise those of eight M=1 calls)

`value` is the step's algorithmic bytes (INT4 codes + bf16 scales/biases + activations in +
outputs, each counted once) divided by the measured step time: whole-job HBM GB/s with every
input already resident. Rotating weight copies and the 438 MB of LM-head traffic per step keep
each call's weights out of the 256 MB last-level cache between uses.

Also printed in the same JSON line:
  roofline      the M=1 LM head (its GEMV kernel and the small argmax reduction kernel), the
                dominant HBM-bound call, against 8 TB/s, its average duration from fence-free HIP
                events on the launch stream around that call in every timed step;
  roofline_moe  the MoE decode call (its three launches) against 8 TB/s, timed the same way;
  roofline_m8   the M=8 LM head on the bit-exact multi-row arm (int8 matrix cores, two launches
                with the argmax reduction) against 8 TB/s, timed the same way;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload (rank 0);
  calls         per-call microseconds and GB/s from a separate pass: batches of back-to-back
                launches between fence-free HIP events (median over batches);
  diagnostics   each call with a cold last-level cache (1 GiB of ordinary reads before every timed call;
                median, p10, p90 of 50), the empty-kernel launch floor, the cost of one grid-wide
                barrier inside a launch (what fusing dependent kernels would pay instead of a
                launch), the HBM read ceiling of
                a plain streaming-read kernel, and the M=1 GEMV's GB/s against its row count.

`--oracle-timing` instead times the fp64 oracle per workload on all cores and on one core.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "lmhead_gemv_m1_counters.json")
# every file the dominant kernel is compiled from (its source, the device helpers and declarations
# it includes, and the build script that holds the compiler flags)
DOMINANT_SRCS = ("hyper_connections_amd/csrc/gemv.hip", "hyper_connections_amd/csrc/dhp_internal.hpp",
                 "include/decodehp.h", "hyper_connections_amd/build.py")


# the same for the other calls whose HBM traffic the counters measured (profiles/traffic_counters.json)
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CALL_SRCS = {
    "lmhead8": ("hyper_connections_amd/csrc/gemv_rows.hip", "hyper_connections_amd/csrc/gemv.hip",
                "hyper_connections_amd/csrc/dhp_internal.hpp", "include/decodehp.h", "hyper_connections_amd/build.py"),
    "moe": ("hyper_connections_amd/csrc/moe.hip", "hyper_connections_amd/csrc/dhp_internal.hpp", "include/decodehp.h",
            "hyper_connections_amd/build.py"),
}


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for rel in paths:
        h.update(rel.encode() + b"\0")
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def dominant_sources_sha256() -> str:
    return sources_sha256(DOMINANT_SRCS)


def call_traffic(call: str):
    """HBM bytes per call from the committed counter runs, if taken on the current sources of
    every kernel of the call; else None."""
    try:
        d = json.load(open(TRAFFIC_PROFILE))["calls"][call]
        if d.get("sources_sha256") != sources_sha256(CALL_SRCS[call]):
            return None
        return d.get("hbm_bytes_per_call")
    except Exception:
        return None


def int4_bytes(rows, cols):
    return rows * cols // 2 + 4 * rows * (cols // 64)


def algorithmic_bytes():
    """Bytes each call must move at least once (weights incl. scales/biases, inputs, outputs)."""
    K = 2560
    b = {}
    b["gemv"] = int4_bytes(2560, K) + 2 * K + 2 * 2560
    C, H, R = 4, 2560, 320
    b["hc"] = (int4_bytes(R, C * H) + int4_bytes(C * H, R) + int4_bytes(C, C * H) + 2 * C * H + 2 * C * H
               + 2 * H + 4 * C) + (2 * C * H * 2 + 2 * H + 4 * C)
    # an inject fused in front of the next read: the residual is read once, the injected one
    # written once, plus the sublayer output and both gate sets
    b["hc_inject_read"] = (int4_bytes(R, C * H) + int4_bytes(C * H, R) + int4_bytes(C, C * H) + 2 * C * H + 2 * H
                           + 4 * C + 2 * C * H + 2 * C * H + 2 * H + 4 * C)
    E, inter, top_k = 256, 512, 8
    b["moe"] = (2 * E * K + 2 * K + (top_k + 1) * (2 * int4_bytes(inter, K) + int4_bytes(K, inter))
                + 2 * K + 2 * K + 8 * top_k)
    b["prefill"] = int4_bytes(8192, K) + 2 * 128 * K + 2 * 128 * 8192
    V = 151936
    # the INT8-router variant at top-10: int8 router codes, bf16 per-element and fp32 per-expert
    # scales, eleven experts (ten routed + the shared one)
    b["moe_i8k10"] = (E * K + 2 * K + 4 * E + 2 * K + 11 * (2 * int4_bytes(inter, K) + int4_bytes(K, inter))
                      + 2 * K + 2 * K + 8 * 10)
    b["lmhead1"] = int4_bytes(V, K) + 2 * K + 4 * V + 4
    b["lmhead8"] = b["lmhead8_mc"] = int4_bytes(V, K) + 2 * 8 * K + 4 * 8 * V + 4 * 8
    # entry replication, the attn and mlp reads (with inject weights) and injects, the stand-in
    # sublayer GEMV, the MoE layer, and the final mixer's read
    read = int4_bytes(R, C * H) + int4_bytes(C * H, R) + int4_bytes(C, C * H) + 4 * C * H + 2 * H + 4 * C
    inject = 4 * C * H + 2 * H + 4 * C
    mixer = int4_bytes(R, C * H) + int4_bytes(C * H, R) + 4 * C * H + 2 * H
    layer = 2 * H + 2 * C * H + 2 * (read + inject) + b["gemv"] + b["moe"] + mixer
    b["layer_eager"] = b["layer_graph"] = layer
    # a 128-token chunk's read (weights once; raw, hc_norm, mixed, gates) and inject
    m = MOE_CHUNK
    b["hc_chunk"] = (int4_bytes(R, C * H) + int4_bytes(C * H, R) + int4_bytes(C, C * H) + 2 * C * H
                     + m * (2 * C * H + 2 * H + 4 * C) + m * (4 * C * H + 2 * H + 4 * C))
    return b


STEP_CALLS = ("gemv", "hc", "moe", "prefill", "lmhead1", "lmhead8")
# Timed per call but outside the step: a 128-token chunk through the same MoE layer, the MoE
# layer with the INT8 scaled router at top-10, an inject fused in front of the next
# hyper-connection read (decodehp_hc_inject_read), the hyper-connection read and inject of a
# 128-token chunk, and one token through a whole decoder layer plus the final mixer, as a
# launch sequence and as a graph; and the M=8 LM head on the matrix-core arm (an explicit option:
# fp16-rounded weights, another summation order).
EXTRA_CALLS = ("moe_prefill", "moe_i8k10", "hc_inject_read", "hc_chunk", "layer_eager", "layer_graph",
               "lmhead8_mc")
CALLS = STEP_CALLS + EXTRA_CALLS
MOE_CHUNK = 128


def moe_prefill_bytes(distinct_experts: int, m: int = MOE_CHUNK) -> int:
    """Algorithmic bytes of one chunk call: the router and shared gate row, every expert the chunk
    routes to once (gate, up and down) plus the shared expert, the chunk's activations in and
    outputs out, ids and weights."""
    K, E, inter, top_k = 2560, 256, 512, 8
    expert = 2 * int4_bytes(inter, K) + int4_bytes(K, inter)
    return 2 * E * K + 2 * K + (distinct_experts + 1) * expert + 2 * m * K * 2 + 8 * m * top_k


def build_workload(torch, hca, synth, ring: int, only=None):
    """Device inputs for every call (or only the call named), with `ring` rotating copies of the
    small weight sets."""
    dev = "cuda"
    t0 = time.time()
    W = {}

    def want(*names):
        return only is None or only in names

    def up_int4(t):
        return hca.Int4Weight.from_logical(t.q, t.s_bits, t.b_bits, dev)

    def clone(w):
        return hca.Int4Weight(w.codes.clone(), w.scales.clone(), w.biases.clone(), w.rows, w.cols)

    if want("gemv"):
        g = synth.gemv_workload(0)
        w0 = up_int4(g["w"])
        W["gemv_w"] = [w0] + [clone(w0) for _ in range(ring - 1)]
        W["gemv_x"] = torch.from_numpy(g["x"]).to(dev)
        W["gemv_y"] = torch.empty(2560, dtype=torch.float16, device=dev)

    if want("hc", "hc_inject_read"):
        h = synth.hc_workload(0)
        hw = (up_int4(h["down"]), up_int4(h["up"]), up_int4(h["inject"]))
        W["hc_w"] = [hw] + [tuple(clone(w) for w in hw) for _ in range(ring - 1)]
        W["hc_wide"] = torch.from_numpy(h["raw"]).to(dev)
        W["hc_gamma"] = hca.bf16_bits_to_tensor(h["gamma_bits"]).to(dev)
        W["hc_out"] = torch.from_numpy(h["out"]).to(dev)
        W["hc_mixed"] = torch.empty(2560, dtype=torch.float16, device=dev)
        W["hc_iw"] = torch.from_numpy(h["iw"]).to(dev)
        W["hc_hidden"] = torch.empty(4 * 2560, dtype=torch.float16, device=dev)
        W["hc_iw_next"] = torch.empty(4, dtype=torch.float32, device=dev)

    if want("moe", "moe_prefill", "moe_i8k10"):
        _moe_workload(torch, hca, synth, W, dev)
    if want("prefill"):
        p = synth.prefill_workload(0)
        p0 = up_int4(p["w"])
        W["pre_w"] = [p0] + [clone(p0) for _ in range(ring - 1)]
        W["pre_x"] = torch.from_numpy(p["x"]).to(dev)
        W["pre_y"] = torch.empty((128, 8192), dtype=torch.float16, device=dev)

    if want("layer_eager", "layer_graph"):
        _layer_workload(torch, hca, synth, W, dev)

    if want("hc_chunk"):
        h = synth.hc_workload(0)
        rows = np.concatenate([h["raw"][None], synth.normal_f16(np.random.default_rng([64, 0]),
                                                                  (MOE_CHUNK - 1, 4 * 2560))])
        W["hcc"] = dict(w=(up_int4(h["down"]), up_int4(h["up"]), up_int4(h["inject"])),
                        gamma=hca.bf16_bits_to_tensor(h["gamma_bits"]).to(dev),
                        raw=torch.from_numpy(rows).to(dev),
                        out=torch.from_numpy(synth.normal_f16(np.random.default_rng([64, 1]),
                                                              (MOE_CHUNK, 2560))).to(dev),
                        mixed=torch.empty((MOE_CHUNK, 2560), dtype=torch.float16, device=dev),
                        iw=torch.empty((MOE_CHUNK, 4), dtype=torch.float32, device=dev))

    if want("lmhead1", "lmhead8", "lmhead8_mc"):
        l1 = synth.lmhead_workload(0, m=1)
        lw = up_int4(l1["w"])
        # four copies: the M=1 call alternates between 0 and 2, the M=8 calls between 1 and 3, so no
        # LM-head call finds the weights it read one step earlier in the 256 MB last-level cache
        W["lm_w"] = [lw, clone(lw), clone(lw), clone(lw)]
        W["lm_x1"] = torch.from_numpy(l1["x"]).to(dev)
        W["lm_x8"] = torch.from_numpy(synth.lmhead_x(0, 8)).to(dev)
        W["lm_y1"] = torch.empty((1, 151936), dtype=torch.float32, device=dev)
        W["lm_y8"] = torch.empty((8, 151936), dtype=torch.float32, device=dev)
        W["lm_a1"] = torch.empty(1, dtype=torch.int32, device=dev)
        W["lm_a8"] = torch.empty(8, dtype=torch.int32, device=dev)
        del l1
    torch.cuda.synchronize()
    print(f"[bench] workload resident in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    return W


def _moe_workload(torch, hca, synth, W, dev):
    def up_int4(t):
        return hca.Int4Weight.from_logical(t.q, t.s_bits, t.b_bits, dev)

    m = synth.moe_workload(0)
    ex = m["experts"]
    W["moe"] = dict(
        gate=hca.Int4Experts.from_logical([e["gate"] for e in ex], dev),
        up=hca.Int4Experts.from_logical([e["up"] for e in ex], dev),
        down=hca.Int4Experts.from_logical([e["down"] for e in ex], dev),
        sg=up_int4(m["shared"]["gate"]), su=up_int4(m["shared"]["up"]), sd=up_int4(m["shared"]["down"]),
        router=hca.bf16_bits_to_tensor(m["router_bits"]).to(dev),
        sgate=hca.bf16_bits_to_tensor(m["sgate_bits"]).to(dev))
    xs = np.concatenate([m["x"][None], synth.moe_x_ring(0, MOE_CHUNK - 1)])
    W["moe_x"] = torch.from_numpy(xs).to(dev)
    W["moe_out"] = torch.empty(2560, dtype=torch.float16, device=dev)
    W["moe_ids"] = torch.empty(8, dtype=torch.int32, device=dev)
    W["moe_w"] = torch.empty(8, dtype=torch.float32, device=dev)
    v = synth.router_variant(0, 256, 2560)
    W["moe"]["router_i8"] = hca.Router(torch.from_numpy(v["codes"]).to(dev),
                                       hca.bf16_bits_to_tensor(v["elem_scale_bits"]).to(dev),
                                       torch.from_numpy(v["expert_scale"]).to(dev))
    W["moe_ids10"] = torch.empty(10, dtype=torch.int32, device=dev)
    W["moe_w10"] = torch.empty(10, dtype=torch.float32, device=dev)
    W["moep_out"] = torch.empty((MOE_CHUNK, 2560), dtype=torch.float16, device=dev)
    W["moep_ids"] = torch.empty((MOE_CHUNK, 8), dtype=torch.int32, device=dev)
    W["moep_w"] = torch.empty((MOE_CHUNK, 8), dtype=torch.float32, device=dev)


def _layer_workload(torch, hca, synth, W, dev):
    d = synth.decode_layer_workload(0, n_layers=1)

    def w4(t):
        return hca.Int4Weight.from_logical(t.q, t.s_bits, t.b_bits, dev)

    def block(b):
        return hca.HcBlock(hca.bf16_bits_to_tensor(b["gamma_bits"]).to(dev), w4(b["down"]), w4(b["up"]),
                           w4(b["inject"]) if b["inject"] is not None else None)

    L = d["layers"][0]
    m = L["moe"]
    ex = m["experts"]
    layer = hca.DecodeLayer(block(L["attn"]), w4(L["stub"]), block(L["mlp"]),
                            hca.bf16_bits_to_tensor(m["router_bits"]).to(dev),
                            hca.bf16_bits_to_tensor(m["sgate_bits"]).to(dev),
                            hca.Int4Experts.from_logical([e["gate"] for e in ex], dev),
                            hca.Int4Experts.from_logical([e["up"] for e in ex], dev),
                            hca.Int4Experts.from_logical([e["down"] for e in ex], dev),
                            w4(m["shared"]["gate"]), w4(m["shared"]["up"]), w4(m["shared"]["down"]), m["top_k"])
    W["layer"] = dict(layers=[layer], mixer=block(d["mixer"]), C=d["C"], H=d["H"],
                      x=torch.from_numpy(d["x"]).to(dev),
                      hidden=torch.empty(d["C"] * d["H"], dtype=torch.float16, device=dev),
                      mixed=torch.empty(d["H"], dtype=torch.float16, device=dev),
                      xg=torch.from_numpy(d["x"]).to(dev),
                      hg=torch.empty(d["C"] * d["H"], dtype=torch.float16, device=dev),
                      mg=torch.empty(d["H"], dtype=torch.float16, device=dev))


def prepare_calls(hca, W, ring: int, only=None):
    """calls[name][i] for ring position i (the MoE token ring has its own length)."""
    C, H = 4, 2560
    make = {
        "gemv": lambda: [hca.prepare_gemv(W["gemv_w"][i], W["gemv_x"], W["gemv_y"]) for i in range(ring)],
        "hc": lambda: [(hca.prepare_hc_read(W["hc_wide"], W["hc_gamma"], C, H, *W["hc_w"][i], W["hc_mixed"],
                                            W["hc_iw"]),
                        hca.prepare_hc_inject(W["hc_wide"], W["hc_out"], W["hc_iw"], C, H)) for i in range(ring)],
        "hc_inject_read": lambda: [hca.prepare_hc_inject_read(W["hc_wide"], W["hc_out"], W["hc_iw"], W["hc_hidden"],
                                                              W["hc_gamma"], C, H, *W["hc_w"][i], W["hc_mixed"],
                                                              W["hc_iw_next"]) for i in range(ring)],
        "moe": lambda: [hca.prepare_moe(W["moe_x"][t], W["moe"]["router"], W["moe"]["sgate"], W["moe"]["gate"],
                                        W["moe"]["up"], W["moe"]["down"], W["moe"]["sg"], W["moe"]["su"],
                                        W["moe"]["sd"], 8, W["moe_out"], W["moe_ids"], W["moe_w"])
                        for t in range(W["moe_x"].shape[0])],
        "moe_i8k10": lambda: [hca.prepare_moe(W["moe_x"][t], W["moe"]["router_i8"], W["moe"]["sgate"],
                                              W["moe"]["gate"], W["moe"]["up"], W["moe"]["down"], W["moe"]["sg"],
                                              W["moe"]["su"], W["moe"]["sd"], 10, W["moe_out"], W["moe_ids10"],
                                              W["moe_w10"]) for t in range(W["moe_x"].shape[0])],
        "moe_prefill": lambda: [hca.prepare_moe_prefill(W["moe_x"], W["moe"]["router"], W["moe"]["sgate"],
                                                        W["moe"]["gate"], W["moe"]["up"], W["moe"]["down"],
                                                        W["moe"]["sg"], W["moe"]["su"], W["moe"]["sd"], 8,
                                                        W["moep_out"], W["moep_ids"], W["moep_w"])],
        "prefill": lambda: [hca.prepare_gemm_batched(W["pre_w"][i], W["pre_x"], W["pre_y"]) for i in range(ring)],
        "hc_chunk": lambda: [(hca.prepare_hc_read_batched(W["hcc"]["raw"], W["hcc"]["gamma"], C, H, *W["hcc"]["w"],
                                                          W["hcc"]["mixed"], W["hcc"]["iw"]),
                              hca.prepare_hc_inject_batched(W["hcc"]["raw"], W["hcc"]["out"], W["hcc"]["iw"], C, H))],
        "layer_eager": lambda: [hca.prepare_decode_layers(W["layer"]["x"], W["layer"]["C"], W["layer"]["H"],
                                                          W["layer"]["layers"], W["layer"]["mixer"],
                                                          W["layer"]["hidden"], W["layer"]["mixed"])],
        "layer_graph": lambda: [hca.LayerGraph(W["layer"]["xg"], W["layer"]["C"], W["layer"]["H"],
                                               W["layer"]["layers"], W["layer"]["mixer"], W["layer"]["hg"],
                                               W["layer"]["mg"]).launch],
        "lmhead1": lambda: [hca.prepare_gemv(W["lm_w"][i], W["lm_x1"], W["lm_y1"], argmax=W["lm_a1"]) for i in (0, 2)],
        "lmhead8": lambda: [hca.prepare_gemv(W["lm_w"][i], W["lm_x8"], W["lm_y8"], argmax=W["lm_a8"]) for i in (1, 3)],
        "lmhead8_mc": lambda: [hca.prepare_gemv(W["lm_w"][i], W["lm_x8"], W["lm_y8"], argmax=W["lm_a8"],
                                                matrix_cores=True) for i in (1, 3)],
    }
    return {name: f() for name, f in make.items() if only is None or name == only}


def chunk_bytes(torch, W, calls) -> int:
    """Run the chunk call once and size it by the distinct experts its routing selected."""
    run_call(calls["moe_prefill"][0])
    torch.cuda.synchronize()
    return moe_prefill_bytes(int(torch.unique(W["moep_ids"]).numel()))


def run_call(c):
    if isinstance(c, tuple):
        for f in c:
            f()
    else:
        c()


def step(calls, i, ev=None, stream=None):
    run_call(calls["gemv"][i % len(calls["gemv"])])
    run_call(calls["hc"][i % len(calls["hc"])])
    if ev is not None:
        ev[0].record(stream)
    run_call(calls["moe"][i % len(calls["moe"])])
    if ev is not None:
        ev[1].record(stream)
    run_call(calls["prefill"][i % len(calls["prefill"])])
    if ev is not None:
        ev[2].record(stream)
    run_call(calls["lmhead1"][i % len(calls["lmhead1"])])
    if ev is not None:
        ev[3].record(stream)
    run_call(calls["lmhead8"][i % len(calls["lmhead8"])])
    if ev is not None:
        ev[4].record(stream)


class HipEvent:
    """A HIP event created without the system-scope fence torch's timing events carry (that fence
    writes back and invalidates caches at every record and adds microseconds to a short call).
    Recorded on the given stream through the HIP runtime the process already loaded."""

    _rt = None

    @classmethod
    def runtime(cls):
        if cls._rt is None:
            import ctypes
            path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
            rt = ctypes.CDLL(path)
            rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._rt = rt
        return cls._rt

    def __init__(self):
        import ctypes
        self.h = ctypes.c_void_p()
        if self.runtime().hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000) != 0:   # hipEventDisableSystemFence
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        import ctypes
        if self.runtime().hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def us_until(self, end) -> float:
        import ctypes
        rt = self.runtime()
        ms = ctypes.c_float()
        if rt.hipEventSynchronize(end.h) != 0 or rt.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    def __del__(self):
        if self._rt is not None and self.h:
            self._rt.hipEventDestroy(self.h)


def per_call_pass(torch, calls, nbytes, iters: int, exact: bool = False):
    """Each call type alone: batches of back-to-back launches (cycling the call's ring) between two
    fence-free events; microseconds per call = batch time / batch size, median (and p10/p90) over
    the batches. `iters` launches in total per call type (the LM heads a quarter of that unless
    `exact`)."""
    out = {}
    stream = torch.cuda.current_stream()
    for name in calls:
        seq = calls[name]
        big = name.startswith("lmhead")
        n = iters if exact else (max(iters, len(seq)) if not big else max(8, iters // 4))
        batch = max(1, min(n, 4 if big else 16))
        nb = max(1, n // batch)
        for i in range(3):
            run_call(seq[i % len(seq)])
        torch.cuda.synchronize()
        us = []
        k = 0
        for _ in range(nb):
            e0, e1 = HipEvent(), HipEvent()
            e0.record(stream)
            for _ in range(batch):
                run_call(seq[k % len(seq)])
                k += 1
            e1.record(stream)
            us.append(e0.us_until(e1) / batch)
        us = np.array(us)
        med = float(np.median(us))
        out[name] = {"launches": nb * batch, "batch": batch, "us": round(med, 2),
                     "p10_us": round(float(np.percentile(us, 10)), 2),
                     "p90_us": round(float(np.percentile(us, 90)), 2),
                     "GBps": round(nbytes[name] / med / 1e3, 1),
                     "pct_hbm_peak": round(100.0 * nbytes[name] / med / 1e3 / HBM_PEAK_GBS, 1)}
    return out


def single_call_latency(torch, calls, names, reps: int = 30):
    """One call at a time onto an idle GPU: synchronize, record, call, record, synchronize; the
    event interval then includes any time the GPU waits for the host to enqueue the next launch.
    Median microseconds over `reps`."""
    stream = torch.cuda.current_stream()
    out = {}
    for name in names:
        seq = calls[name]
        us = []
        for i in range(reps + 3):
            torch.cuda.synchronize()
            e0, e1 = HipEvent(), HipEvent()
            e0.record(stream)
            run_call(seq[i % len(seq)])
            e1.record(stream)
            t = e0.us_until(e1)
            if i >= 3:
                us.append(t)
        out[name] = round(float(np.median(us)), 2)
    return out


FLUSH_BYTES = 1 << 30          # a read of 1 GiB (more than 4x the 256 MB last-level cache) evicts it


def _stats(us):
    us = np.asarray(us)
    return {"us": round(float(np.median(us)), 2), "p10_us": round(float(np.percentile(us, 10)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2)}


def flush_llc(torch, flush):
    """Evict the last-level cache: 1 GiB of ordinary (caching) reads. The read probe's streaming
    loads do not displace it: after a 1 GiB probe read the M=1 LM head still found much of its
    219 MB of weights there (38 us, against 43 us after ordinary reads)."""
    flush.view(torch.float32).sum()


def cold_call_pass(torch, hca, calls, nbytes, flush, sink, reps: int = 50):
    """Each call with a cold last-level cache: 1 GiB of ordinary reads before every timed call
    (flush_llc), then fence-free events on the stream bracket the call alone. Median and p10/p90
    over `reps` calls (cycling each call's weight copies)."""
    stream = torch.cuda.current_stream()
    out = {}
    for name, seq in calls.items():
        run_call(seq[0])
        evs = []
        for i in range(reps):
            flush_llc(torch, flush)
            e0, e1 = HipEvent(), HipEvent()
            e0.record(stream)
            run_call(seq[i % len(seq)])
            e1.record(stream)
            evs.append((e0, e1))
        st = _stats([a.us_until(b) for a, b in evs])
        out[name] = {**st, "GBps": round(nbytes[name] / st["us"] / 1e3, 1),
                     "pct_hbm_peak": round(100.0 * nbytes[name] / st["us"] / 1e3 / HBM_PEAK_GBS, 1)}
    return out


def launch_floor(torch, hca, n: int = 200, reps: int = 30):
    """The empty kernel: n launches back to back from one library call (no host work between
    them) between two events, the same n launched one library call each from Python (what the
    per-call pass pays per launch), and one launch onto an idle GPU (median over reps)."""
    stream = torch.cuda.current_stream()
    hca.probe_empty(10)
    torch.cuda.synchronize()
    e0, e1 = HipEvent(), HipEvent()
    e0.record(stream)
    hca.probe_empty(n)
    e1.record(stream)
    b2b = e0.us_until(e1) / n
    torch.cuda.synchronize()
    e0, e1 = HipEvent(), HipEvent()
    e0.record(stream)
    for _ in range(n):
        hca.probe_empty()
    e1.record(stream)
    py = e0.us_until(e1) / n
    single = []
    for _ in range(reps):
        torch.cuda.synchronize()
        a, b = HipEvent(), HipEvent()
        a.record(stream)
        hca.probe_empty()
        b.record(stream)
        single.append(a.us_until(b))
    return {"back_to_back_us": round(b2b, 2), "one_python_call_each_us": round(py, 2),
            "single_idle_us": round(float(np.median(single)), 2)}


def grid_barrier_cost(torch, hca, reps: int = 10):
    """Microseconds per grid-wide barrier inside one launch (the slope between launches with 1 and
    21 barriers), for 64 and 256 blocks, ordered (release/acquire, as data hand-over between blocks
    needs) and relaxed, next to the kernel boundary it would replace (launch_floor)."""
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    out = {}
    for blocks in (64, cus):
        for ordered in (True, False):
            t = {}
            for n in (1, 21):
                hca.probe_grid_barrier(blocks, n, ordered, state, sink)
                torch.cuda.synchronize()
                a, b = HipEvent(), HipEvent()
                a.record(stream)
                for _ in range(reps):
                    hca.probe_grid_barrier(blocks, n, ordered, state, sink)
                b.record(stream)
                t[n] = a.us_until(b) / reps
            out[f"{'ordered' if ordered else 'relaxed'}_{blocks}_blocks_us"] = round((t[21] - t[1]) / 20, 2)
    torch.cuda.synchronize()
    st = state.cpu().tolist()
    out["all_waits_ended"] = bool(st[0] == 0 and st[2] == 0)
    return out


def read_ceiling(torch, hca, flush, sink, target_bytes: int = 219400704, reps: int = 5):
    """The read probe over a 1 GiB buffer (larger than the last-level cache, so every pass reads
    HBM) for a grid of (blocks per CU, loads in flight per lane), and the best arrangement over a
    buffer of the M=1 LM head's size, flushed before each pass."""
    stream = torch.cuda.current_stream()
    grid = {}
    for bpc in (1, 2, 4, 8):
        for u in (2, 4, 8):
            hca.probe_read(flush, bpc, u, sink)
            e0, e1 = HipEvent(), HipEvent()
            e0.record(stream)
            for _ in range(reps):
                hca.probe_read(flush, bpc, u, sink)
            e1.record(stream)
            grid[f"{bpc}x{u}"] = round(FLUSH_BYTES * reps / e0.us_until(e1) / 1e3, 1)
    best = max(grid, key=grid.get)
    bpc, u = (int(v) for v in best.split("x"))
    target = torch.empty(target_bytes, dtype=torch.uint8, device="cuda")
    us = []
    for _ in range(reps * 4):
        flush_llc(torch, flush)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        hca.probe_read(target, bpc, u, sink)
        e1.record(stream)
        us.append(e0.us_until(e1))
    t = float(np.median(us))
    return {"GBps_1GiB": grid, "best": best, "GBps_best_1GiB": grid[best],
            "GBps_lmhead_size_cold": round(target_bytes / t / 1e3, 1), "lmhead_size_us": round(t, 2)}


def rows_sweep(torch, hca, W, flush, sink, reps: int = 20):
    """M=1 GEMV (fp16 out, no argmax) over the first N rows of the LM-head weight, K = 2560, each
    call after a cache flush: GB/s of algorithmic bytes against N."""
    stream = torch.cuda.current_stream()
    w = W["lm_w"][0]
    x = W["lm_x1"]
    y = torch.empty(w.rows, dtype=torch.float16, device="cuda")
    out = {}
    for n in (2560, 8192, 32768, 65536, 151936):
        wn = hca.Int4Weight(w.codes[:n], w.scales[:n], w.biases[:n], n, w.cols)
        c = hca.prepare_gemv(wn, x, y[:n])
        c()
        us = []
        for _ in range(reps):
            flush_llc(torch, flush)
            e0, e1 = HipEvent(), HipEvent()
            e0.record(stream)
            c()
            e1.record(stream)
            us.append(e0.us_until(e1))
        t = float(np.median(us))
        b = int4_bytes(n, 2560) + 2 * 2560 + 2 * n
        out[str(n)] = {"us": round(t, 2), "GBps": round(b / t / 1e3, 1)}
    return out


def copy_probe(torch):
    """A plain 1 GiB device copy, for scaling the HBM byte counters (FETCH_SIZE / WRITE_SIZE)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / 5
    return {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "us": round(dt * 1e6, 1),
            "GBps_read_plus_write": round(2 * (1 << 30) / dt / 1e9, 1)}


def summarize_profile(path: str, filt: str = ""):
    """Per-kernel figures from rocprofv3 SQLite output under `path`: launch count and mean/min
    duration from a kernel trace, and per-dispatch counter totals (summed over the rows of one
    dispatch, averaged over dispatches) from --pmc runs."""
    import glob
    import sqlite3
    from collections import defaultdict
    trace = defaultdict(list)
    ctr = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    for f in sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(f)
        tables = {r[0] for r in con.execute("select name from sqlite_master where type in ('table','view')")}
        if "kernels" in tables:
            for name, t0, t1 in con.execute("select name, start, end from kernels"):
                if filt in name:
                    trace[name].append((t1 - t0) / 1e3)
        if "counters_collection" in tables:
            for name, cn, val, disp in con.execute(
                    "select kernel_name, counter_name, value, dispatch_id from counters_collection"):
                if filt in name:
                    ctr[name][cn][(f, disp)] += val
        con.close()
    out = {}
    for name, ds in trace.items():
        out.setdefault(name, {})["trace"] = {"launches": len(ds), "avg_us": round(sum(ds) / len(ds), 2),
                                             "min_us": round(min(ds), 2), "total_us": round(sum(ds), 1)}
    for name, cs in ctr.items():
        out.setdefault(name, {})["counters"] = {
            cn: {"dispatches": len(v), "mean": sum(v.values()) / len(v)} for cn, v in sorted(cs.items())}
    return out


def cpu_baseline(synth):
    """The fp64 oracle on a bounded sample of one step, scaled to GB/s of algorithmic bytes."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    K = 2560
    g = synth.gemv_workload(0)
    h = synth.hc_workload(0)
    m = synth.moe_workload(0, with_experts=False)
    sel = {}
    p = synth.prefill_workload(0)
    lw = synth.lmhead_workload(0, m=1)
    x8 = synth.lmhead_x(0, 8)
    PR, LR = 1024, 16384                      # prefill and LM-head row samples
    done = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.dequant_gemv(g["w"].q, g["w"].s_bits, g["w"].b_bits, g["x"])
        done += int4_bytes(2560, K) + 4 * K
        r = oracle.hc_read(h["raw"], h["gamma_bits"], h["down"], h["up"], h["inject"], 4, 2560)
        oracle.hc_inject(h["raw"], h["out"], r["inject_w"], 4, 2560)
        done += algorithmic_bytes()["hc"]
        logits = oracle.router_logits(m["router_bits"], m["x"])
        ids = oracle.select_topk(logits, 8)
        experts = {int(e): sel.setdefault(int(e), synth.moe_expert(0, int(e))) for e in ids}
        oracle.moe_decode(m["x"], m["router_bits"], m["sgate_bits"], m["shared"], experts, 8)
        done += algorithmic_bytes()["moe"]
        oracle.dequant_gemv(p["w"].q[:PR], p["w"].s_bits[:PR], p["w"].b_bits[:PR], p["x"])
        done += int4_bytes(PR, K) + 2 * 128 * K + 2 * 128 * PR
        y1 = oracle.dequant_gemv(lw["w"].q[:LR], lw["w"].s_bits[:LR], lw["w"].b_bits[:LR], lw["x"][0])
        oracle.argmax_lowest(y1)
        done += int4_bytes(LR, K) + 2 * K + 4 * LR
        y8 = oracle.dequant_gemv(lw["w"].q[:LR], lw["w"].s_bits[:LR], lw["w"].b_bits[:LR], x8)
        oracle.argmax_lowest(y8)
        done += int4_bytes(LR, K) + 16 * K + 32 * LR
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 200:      # about 10 s of CPU work
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{reps} pass(es) of one step with the prefill projection cut to {PR} of 8192 rows and "
                       f"both LM-head calls to {LR} of 151936 rows (other calls whole); fp64 NumPy; "
                       f"{dt:.1f} s wall"),
            "seconds": round(dt, 2)}


def oracle_config_timing(synth, reps: int = 3):
    """The fp64 oracle per workload, generation excluded: median wall time of `reps` runs in this
    process (whatever BLAS/OpenMP threads it has)."""
    import oracle
    g = synth.gemv_workload(0)
    h = synth.hc_workload(0)
    m = synth.moe_workload(0, with_experts=False)
    ids = oracle.select_topk(oracle.router_logits(m["router_bits"], m["x"]), 8)
    experts = {int(e): synth.moe_expert(0, int(e)) for e in ids}
    p = synth.prefill_workload(0)
    lw = synth.lmhead_workload(0, m=1)
    x8 = synth.lmhead_x(0, 8)
    work = {
        "gemv_2560": lambda: oracle.dequant_gemv(g["w"].q, g["w"].s_bits, g["w"].b_bits, g["x"]),
        "hc_read_inject": lambda: oracle.hc_inject(
            h["raw"], h["out"],
            oracle.hc_read(h["raw"], h["gamma_bits"], h["down"], h["up"], h["inject"], 4, 2560)["inject_w"], 4, 2560),
        "moe_decode": lambda: oracle.moe_decode(m["x"], m["router_bits"], m["sgate_bits"], m["shared"], experts, 8),
        "prefill_m128": lambda: oracle.dequant_gemv(p["w"].q, p["w"].s_bits, p["w"].b_bits, p["x"]),
        "lmhead_m1": lambda: oracle.argmax_lowest(oracle.dequant_gemv(lw["w"].q, lw["w"].s_bits, lw["w"].b_bits,
                                                                       lw["x"][0])),
        "lmhead_m8": lambda: oracle.argmax_lowest(oracle.dequant_gemv(lw["w"].q, lw["w"].s_bits, lw["w"].b_bits, x8)),
    }
    out = {}
    for name, f in work.items():
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        out[name] = round(float(np.median(ts)), 4)
    return out


def oracle_timing(synth):
    """Per-workload oracle seconds on every core visible to the process, then again in a child
    process limited to one BLAS/OpenMP thread."""
    import subprocess
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    except Exception:
        blas = None
    allc = oracle_config_timing(synth)
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-timing-child"], env=env,
                       capture_output=True, text=True, check=True)
    one = json.loads(r.stdout.strip().splitlines()[-1])
    return {"affinity_cores": len(os.sched_getaffinity(0)), "blas": blas, "seconds_all_cores": allc,
            "seconds_one_core": one, "reps": 3, "note": "median of 3, input generation excluded"}


def traffic_from_profile():
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter runs, if they
    were taken on the current sources of that kernel (every file in DOMINANT_SRCS); else None."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    try:
        d = json.load(open(PROFILE_COUNTERS))
        if d.get("sources_sha256") != dominant_sources_sha256():
            return None
        return d.get("hbm_bytes_per_launch")
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ring", type=int, default=8, help="rotating copies of each small weight set")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-call", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="with --only: evict the last-level cache before every launch (median over launches)")
    ap.add_argument("--copy-probe", action="store_true", help="also time a plain 1 GiB copy (counter scaling)")
    ap.add_argument("--only", choices=CALLS + ("copy",),
                    help="launch just this call (or the plain 1 GiB copy) --steps times after --warmup, and "
                         "print its timing; for profiler runs")
    ap.add_argument("--summarize", metavar="DIR", help="print per-kernel figures from rocprofv3 output in DIR")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="time the fp64 oracle per workload on all cores and on one core (CPU only), print JSON")
    ap.add_argument("--oracle-timing-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--filter", default="", help="kernel-name substring for --summarize")
    args = ap.parse_args()

    if args.summarize:
        print(json.dumps(summarize_profile(args.summarize, args.filter), indent=1))
        return
    if args.oracle_timing or args.oracle_timing_child:
        import synth
        r = oracle_config_timing(synth) if args.oracle_timing_child else oracle_timing(synth)
        print(json.dumps(r), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the decode hot path here runs on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import hyper_connections_amd as hca
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    hca.lib()                                 # fails loudly when the HIP library is not built
    nbytes = algorithmic_bytes()
    step_bytes = sum(nbytes[c] for c in STEP_CALLS)

    if args.only == "copy":
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "launches": args.warmup + args.steps}), flush=True)
        return
    if args.only:
        W = build_workload(torch, hca, synth, args.ring, only=args.only)
        calls = prepare_calls(hca, W, args.ring, only=args.only)
        if args.only == "moe_prefill":
            nbytes["moe_prefill"] = chunk_bytes(torch, W, calls)
        for i in range(args.warmup):
            run_call(calls[args.only][i % len(calls[args.only])])
        if args.cold:
            flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
            r = cold_call_pass(torch, hca, calls, nbytes, flush, None, reps=args.steps)[args.only]
            r["cold"] = True
        else:
            r = per_call_pass(torch, calls, nbytes, iters=args.steps, exact=True)[args.only]
        print(json.dumps({"only": args.only, "algorithmic_bytes": nbytes[args.only], **r}), flush=True)
        return

    W = build_workload(torch, hca, synth, args.ring)
    calls = prepare_calls(hca, W, args.ring)
    nbytes["moe_prefill"] = chunk_bytes(torch, W, calls)

    for i in range(args.warmup):
        step(calls, i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [tuple(HipEvent() for _ in range(5)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(calls, args.warmup + i, ev[i], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    moe_us = float(np.mean([e[0].us_until(e[1]) for e in ev]))
    dom_us = float(np.mean([e[2].us_until(e[3]) for e in ev]))
    m8_us = float(np.mean([e[3].us_until(e[4]) for e in ev]))
    print(f"[bench] {args.steps} steps, {ms_per_step:.3f} ms/step, {value:.1f} GB/s; lmhead1 {dom_us:.2f} us, "
          f"lmhead8 {m8_us:.2f} us",
          file=sys.stderr, flush=True)

    dom_ach = nbytes["lmhead1"] / dom_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(dom_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_ach / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(),
                "kernel": "k_gemv_m1_reg<5,f32,argmax> + k_argmax_final (LM head 151936 x 2560, M=1)",
                "algorithmic_bytes_per_launch": nbytes["lmhead1"], "avg_launch_us": round(dom_us, 2)}
    m8_ach = nbytes["lmhead8"] / m8_us / 1e3
    roofline_m8 = {"bound": "hbm", "achieved": round(m8_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(m8_ach / HBM_PEAK_GBS, 4), "traffic": call_traffic("lmhead8"),
                   "kernel": "k_gemv_rows<2,f32,argmax,full,one> + k_argmax_final (LM head 151936 x 2560, M=8)",
                   "algorithmic_bytes_per_launch": nbytes["lmhead8"], "avg_call_us": round(m8_us, 2)}
    moe_ach = nbytes["moe"] / moe_us / 1e3
    roofline_moe = {"bound": "hbm", "achieved": round(moe_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(moe_ach / HBM_PEAK_GBS, 4), "traffic": call_traffic("moe"),
                    "kernel": "MoE decode (router + top-8, phase 1, phase 2: three launches), E=256, top-8",
                    "algorithmic_bytes_per_launch": nbytes["moe"], "avg_call_us": round(moe_us, 2)}

    per_call = None if args.no_per_call else per_call_pass(torch, calls, nbytes, iters=100)
    if per_call is not None:
        for name, us in single_call_latency(torch, calls, ("layer_eager", "layer_graph")).items():
            per_call[name]["single_call_us"] = us
    diag = None
    if not args.no_per_call:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        sink = torch.empty(16 * 1024, dtype=torch.int32, device="cuda")
        diag = {"calls_cold": cold_call_pass(torch, hca, calls, nbytes, flush, sink),
                "launch_floor": launch_floor(torch, hca),
                "grid_barrier": grid_barrier_cost(torch, hca),
                "read_ceiling": read_ceiling(torch, hca, flush, sink),
                "gemv_rows_sweep_cold": rows_sweep(torch, hca, W, flush, sink)}
        del flush
    probe = copy_probe(torch) if args.copy_probe else None

    cpu = None if args.no_cpu_baseline else cpu_baseline(synth)

    line = {
        "metric": "achieved HBM GB/s (% of peak) and us/call for INT4 dequant GEMV + MoE decode",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4-affine weights; GEMV group sums exact on int8 pieces, f16 operands elsewhere; f32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": "decode hot-path step: gemv 2560x2560 M=1; hc read+inject C=4 H=2560 R=320; "
                               "moe E=256 top-8 hidden 2560 inter 512 + shared; prefill M=128 N=8192 K=2560; "
                               "lm head 151936x2560 M=1 and M=8 with argmax",
                   "step_bytes": step_bytes, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
                   "parallelism": "1 GPU"},
        "roofline": roofline,
        "roofline_m8": roofline_m8,
        "roofline_moe": roofline_moe,
        "cpu_baseline": cpu,
        "calls": per_call,
    }
    if diag:
        line["diagnostics"] = diag
    if probe:
        line["copy_probe"] = probe
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
