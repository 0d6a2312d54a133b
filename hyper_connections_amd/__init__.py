"""Python binding of libdecodehp (MI355X decode hot path).

Argument marshalling only: every step of the path runs in the HIP kernels behind the C
ABI declared in include/decodehp.h. PyTorch supplies device memory and the stream; the
binding checks dtype, device and contiguity, allocates the workspace an entry point asks
for, and raises DecodeHPError on a nonzero return. There is no fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .layout import pack_int4_codes, bf16_bits_to_tensor  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdecodehp.so")

DHP_F16, DHP_F32, DHP_BF16, DHP_I8 = 0, 1, 2, 3
DHP_MOE_MAX_TOP_K = 10
DHP_OP_GEMV_ARGMAX, DHP_OP_MOE_DECODE, DHP_OP_HC_READ = 1, 2, 3
DHP_MOE_FP16_BOUNDARY = 1
ERRORS = {-1: "invalid argument", -2: "unsupported", -3: "misaligned", -4: "workspace",
          -5: "no device", -6: "launch"}


class DecodeHPError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libdecodehp error {code} ({ERRORS.get(code, '?')}): {message}")
        self.code = code


class CInt4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("group", ctypes.c_int32)]


class CInt4Experts(ctypes.Structure):
    _fields_ = [("first", CInt4), ("codes_stride", ctypes.c_int64), ("scales_stride", ctypes.c_int64),
                ("count", ctypes.c_int32)]


P4_, PE_ = ctypes.POINTER(CInt4), ctypes.POINTER(CInt4Experts)


class CRouter(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("elem_scale", ctypes.c_void_p),
                ("expert_scale", ctypes.c_void_p)]


class CHcBlock(ctypes.Structure):
    _fields_ = [("hc_norm", ctypes.c_void_p), ("down", P4_), ("up", P4_), ("inject", P4_)]


class CDecodeLayer(ctypes.Structure):
    _fields_ = [("attn_hc", CHcBlock), ("sublayer", P4_), ("mlp_hc", CHcBlock), ("router", ctypes.c_void_p),
                ("router_dtype", ctypes.c_int32), ("shared_gate_row", ctypes.c_void_p), ("gate", PE_),
                ("up", PE_), ("down", PE_), ("shared_gate", P4_), ("shared_up", P4_), ("shared_down", P4_),
                ("top_k", ctypes.c_int32), ("moe_flags", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdecodehp; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with hyper_connections_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P4, PE = ctypes.POINTER(CInt4), ctypes.POINTER(CInt4Experts)
        L.decodehp_dequant_gemv.argtypes = [P4, vp, i32, vp, i32, vp, vp, sz, vp]
        L.decodehp_dequant_gemv_mc.argtypes = [P4, vp, i32, vp, i32, vp, vp, sz, vp]
        L.decodehp_dequant_gemm_batched.argtypes = [P4, vp, i32, vp, vp]
        L.decodehp_moe_decode.argtypes = [vp, vp, i32, vp, PE, PE, PE, P4, P4, P4, i32, i32, vp, vp, vp,
                                          vp, sz, vp]
        L.decodehp_moe_prefill.argtypes = [vp, i32, vp, i32, vp, PE, PE, PE, P4, P4, P4, i32, i32, vp, vp, vp,
                                           vp, sz, vp]
        PR = ctypes.POINTER(CRouter)
        L.decodehp_moe_decode_ex.argtypes = [vp, PR, vp, PE, PE, PE, P4, P4, P4, i32, i32, vp, vp, vp, vp, sz, vp]
        L.decodehp_moe_prefill_ex.argtypes = [vp, i32, PR, vp, PE, PE, PE, P4, P4, P4, i32, i32, vp, vp, vp, vp,
                                              sz, vp]
        L.decodehp_moe_decode_noalloc.argtypes = [vp, vp, i32, vp, PE, PE, PE, P4, P4, P4, i32, i32, vp, vp, vp,
                                                  vp]
        L.decodehp_moe_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.decodehp_moe_prefill_workspace_bytes.restype = sz
        PL, PB = ctypes.POINTER(CDecodeLayer), ctypes.POINTER(CHcBlock)
        L.decodehp_decode_layers_workspace_bytes.argtypes = [i32, i32, PL, i32, PB]
        L.decodehp_decode_layers_workspace_bytes.restype = sz
        L.decodehp_decode_layers.argtypes = [vp, i32, i32, ctypes.c_float, PL, i32, PB, vp, vp, vp, sz, vp]
        L.decodehp_graph_capture_decode_layers.argtypes = [vp, i32, i32, ctypes.c_float, PL, i32, PB, vp, vp, vp,
                                                           sz, ctypes.POINTER(vp)]
        L.decodehp_graph_launch.argtypes = [vp, vp]
        L.decodehp_graph_destroy.argtypes = [vp]
        L.decodehp_graph_destroy.restype = None
        L.decodehp_hc_read.argtypes = [vp, vp, i32, i32, ctypes.c_float, P4, P4, P4, vp, vp, vp, sz, vp]
        L.decodehp_hc_read_batched.argtypes = [vp, i32, vp, i32, i32, ctypes.c_float, P4, P4, P4, vp, vp, vp, sz,
                                               vp]
        L.decodehp_hc_read_batched_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.decodehp_hc_read_batched_workspace_bytes.restype = sz
        L.decodehp_hc_inject_batched.argtypes = [vp, i32, vp, vp, i32, i32, vp]
        L.decodehp_hc_inject.argtypes = [vp, vp, vp, i32, i32, vp]
        L.decodehp_hc_inject_read.argtypes = [vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, P4, P4, P4, vp, vp, vp,
                                              sz, vp]
        L.decodehp_probe_empty.argtypes = [i32, vp]
        L.decodehp_probe_read.argtypes = [vp, sz, i32, i32, vp, i32, vp]
        L.decodehp_probe_grid_barrier.argtypes = [i32, i32, i32, vp, vp, vp]
        L.decodehp_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.decodehp_workspace_bytes.restype = sz
        L.decodehp_last_error.restype = ctypes.c_char_p
        L.decodehp_version.restype = i32
        for name in ("decodehp_dequant_gemv", "decodehp_dequant_gemv_mc", "decodehp_dequant_gemm_batched",
                     "decodehp_moe_decode",
                     "decodehp_moe_decode_noalloc",
                     "decodehp_moe_prefill", "decodehp_hc_read", "decodehp_hc_inject", "decodehp_decode_layers",
                     "decodehp_hc_inject_read",
                     "decodehp_hc_read_batched", "decodehp_hc_inject_batched",
                     "decodehp_graph_capture_decode_layers", "decodehp_graph_launch"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise DecodeHPError(rc, lib().decodehp_last_error().decode())


def workspace_bytes(op: int, a: int, b: int = 0, c: int = 0) -> int:
    return int(lib().decodehp_workspace_bytes(op, a, b, c))


# --------------------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, dtype, name, numel=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Int4Weight:
    """Device INT4-affine tensor: codes uint8 [rows, cols/2], scales/biases bf16-bit int16 [rows, cols/64]."""

    codes: "object"
    scales: "object"
    biases: "object"
    rows: int
    cols: int

    @classmethod
    def from_logical(cls, q, s_bits, b_bits, device="cuda"):
        torch = _torch()
        q = np.asarray(q)
        rows, cols = q.shape
        codes = torch.from_numpy(pack_int4_codes(q)).to(device)
        scales = bf16_bits_to_tensor(s_bits).to(device)
        biases = bf16_bits_to_tensor(b_bits).to(device)
        return cls(codes, scales, biases, rows, cols)

    def desc(self) -> CInt4:
        torch = _torch()
        _need(self.codes, torch.uint8, "codes", self.rows * self.cols // 2)
        _need(self.scales, torch.int16, "scales", self.rows * self.cols // 64)
        _need(self.biases, torch.int16, "biases", self.rows * self.cols // 64)
        return CInt4(self.codes.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(),
                     self.rows, self.cols, 64)

    @property
    def nbytes(self) -> int:
        return self.rows * self.cols // 2 + 2 * 2 * self.rows * (self.cols // 64)


@dataclass
class Int4Experts:
    """`count` same-shaped INT4 tensors stored back to back: codes [count, rows, cols/2], scales/biases
    [count, rows, cols/64]."""

    codes: "object"
    scales: "object"
    biases: "object"
    count: int
    rows: int
    cols: int

    @classmethod
    def from_logical(cls, tensors, device="cuda"):
        torch = _torch()
        rows, cols = tensors[0].q.shape
        codes = torch.from_numpy(np.stack([pack_int4_codes(t.q) for t in tensors])).to(device)
        scales = torch.from_numpy(np.stack([np.asarray(t.s_bits, np.uint16) for t in tensors]).view(np.int16)).to(device)
        biases = torch.from_numpy(np.stack([np.asarray(t.b_bits, np.uint16) for t in tensors]).view(np.int16)).to(device)
        return cls(codes, scales, biases, len(tensors), rows, cols)

    def desc(self) -> CInt4Experts:
        torch = _torch()
        _need(self.codes, torch.uint8, "expert codes", self.count * self.rows * self.cols // 2)
        _need(self.scales, torch.int16, "expert scales", self.count * self.rows * self.cols // 64)
        _need(self.biases, torch.int16, "expert biases", self.count * self.rows * self.cols // 64)
        first = CInt4(self.codes.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(),
                      self.rows, self.cols, 64)
        return CInt4Experts(first, self.rows * self.cols // 2, 2 * self.rows * (self.cols // 64), self.count)


_ws_cache = {}


def _workspace(nbytes: int, device, kind: str = "scratch", stream=None):
    """Per (device, stream, kind) workspace, grown on demand. It is allocated on the stream the
    call runs on, so that when a grown workspace replaces it, torch's caching allocator hands the
    old memory only to later work on that same stream."""
    torch = _torch()
    if nbytes == 0:
        return None
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (str(device), s.cuda_stream, kind)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


# --------------------------------------------------------------------------- entry points

def dequant_gemv(w: Int4Weight, x, y=None, out_dtype=None, argmax=False, stream=None, matrix_cores=False):
    """y[m, n] = sum_k W[n, k] x[m, k]; x fp16 [K] or [m, K] (m <= 16). Returns y (and argmax int32 [m]).
    matrix_cores: the matrix-core arm (decodehp_dequant_gemv_mc), not bit-equal to per-row calls."""
    torch = _torch()
    out_dtype = out_dtype or torch.float16
    x2 = x.reshape(-1, w.cols)
    m = x2.shape[0]
    _need(x2, torch.float16, "x")
    if y is None:
        y = torch.empty((m, w.rows), dtype=out_dtype, device=x.device)
    _need(y, out_dtype, "y", m * w.rows)
    am = torch.empty(m, dtype=torch.int32, device=x.device) if argmax else None
    ws = _workspace(workspace_bytes(DHP_OP_GEMV_ARGMAX, w.rows, m), x.device, "argmax", stream=stream) if argmax else None
    d = w.desc()
    fn = lib().decodehp_dequant_gemv_mc if matrix_cores else lib().decodehp_dequant_gemv
    _check(fn(ctypes.byref(d), x2.data_ptr(), m, y.data_ptr(),
                                       DHP_F32 if out_dtype == torch.float32 else DHP_F16,
                                       _ptr(am), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    yv = y.reshape(x.shape[:-1] + (w.rows,)) if x.dim() == 1 else y
    return (yv, am) if argmax else yv


def dequant_gemm_batched(w: Int4Weight, x, y=None, stream=None):
    """Y = X W^T for X fp16 [m, K] (m <= 128); Y fp16 [m, N]."""
    torch = _torch()
    _need(x, torch.float16, "x")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.rows), dtype=torch.float16, device=x.device)
    _need(y, torch.float16, "y", m * w.rows)
    d = w.desc()
    _check(lib().decodehp_dequant_gemm_batched(ctypes.byref(d), x.data_ptr(), m, y.data_ptr(), _stream(stream)))
    return y


class Router:
    """A router with the optional scales of the _ex entry points.

    weights [E, hidden]: bf16 bits (int16), float32, or int8 codes; elem_scale: bf16 bits (int16)
    [hidden] that multiply x before the dot products, or None; expert_scale: float32 [E] that
    multiplies each selected expert's routing weight after the softmax, or None.
    """

    def __init__(self, weights, elem_scale=None, expert_scale=None):
        torch = _torch()
        kinds = {torch.int16: DHP_BF16, torch.float32: DHP_F32, torch.int8: DHP_I8}
        if weights.dtype not in kinds:
            raise TypeError("router weights: int16 (bf16 bits), float32 or int8")
        self.weights, self.dtype = weights, kinds[weights.dtype]
        self.elem_scale, self.expert_scale = elem_scale, expert_scale

    def desc(self, n_experts: int, hidden: int) -> CRouter:
        torch = _torch()
        _need(self.weights, self.weights.dtype, "router", n_experts * hidden)
        if self.elem_scale is not None:
            _need(self.elem_scale, torch.int16, "elem_scale", hidden)
        if self.expert_scale is not None:
            _need(self.expert_scale, torch.float32, "expert_scale", n_experts)
        return CRouter(self.weights.data_ptr(), self.dtype, _ptr(self.elem_scale), _ptr(self.expert_scale))


def _plain_router(router, n_experts, hidden):
    torch = _torch()
    if router.dtype == torch.int16:
        rdt = DHP_BF16
    elif router.dtype == torch.float32:
        rdt = DHP_F32
    else:
        raise TypeError("router: int16 (bf16 bits) or float32 (int8 routers go through Router)")
    _need(router, router.dtype, "router", n_experts * hidden)
    return rdt


def _moe_args(x, m, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k, out, ids,
              weights, fp16_boundary, stream):
    """(entry point, its arguments, what must stay alive) of one MoE call; m None: the decode
    entry points (one token), else the prefill ones over m tokens."""
    torch = _torch()
    hidden, rows = gate.cols, 1 if m is None else m
    _need(x, torch.float16, "x", rows * hidden)
    _need(shared_gate_row, torch.int16, "shared_gate_row", hidden)
    _need(out, torch.float16, "out", rows * hidden)
    _need(ids, torch.int32, "ids", rows * top_k)
    _need(weights, torch.float32, "weights", rows * top_k)
    if m is None:
        ws = _workspace(workspace_bytes(DHP_OP_MOE_DECODE, gate.count, top_k, gate.rows), x.device, stream=stream)
    else:
        ws = _workspace(moe_prefill_workspace_bytes(m, gate.count, top_k, gate.rows, hidden), x.device, "moe_prefill", stream=stream)
    descs = (gate.desc(), up.desc(), down.desc(), shared_gate.desc(), shared_up.desc(), shared_down.desc())
    if isinstance(router, Router):
        rd = router.desc(gate.count, hidden)
        head, keep_r = (ctypes.byref(rd),), rd
        fn = lib().decodehp_moe_decode_ex if m is None else lib().decodehp_moe_prefill_ex
    else:
        head, keep_r = (router.data_ptr(), _plain_router(router, gate.count, hidden)), None
        fn = lib().decodehp_moe_decode if m is None else lib().decodehp_moe_prefill
    args = (x.data_ptr(), *(() if m is None else (m,)), *head, shared_gate_row.data_ptr(),
            *[ctypes.byref(d) for d in descs], top_k, DHP_MOE_FP16_BOUNDARY if fp16_boundary else 0,
            out.data_ptr(), ids.data_ptr(), weights.data_ptr(), _ptr(ws), 0 if ws is None else ws.numel(),
            _stream(stream))
    keep = (descs, keep_r, x, router, shared_gate_row, out, ids, weights, ws, gate, up, down, shared_gate, shared_up,
            shared_down)
    return fn, args, keep


def moe_decode(x, router, shared_gate_row, gate: Int4Experts, up: Int4Experts, down: Int4Experts,
               shared_gate: Int4Weight, shared_up: Int4Weight, shared_down: Int4Weight, top_k: int,
               fp16_boundary=False, out=None, ids=None, weights=None, stream=None):
    """One token through the routed MoE layer. router: bf16 bits (int16) or fp32 [E, hidden], or a
    Router (int8 codes and/or scales).

    Returns (out fp16 [hidden], ids int32 [top_k], weights fp32 [top_k]).
    """
    torch = _torch()
    dev = x.device
    out = torch.empty(gate.cols, dtype=torch.float16, device=dev) if out is None else out
    ids = torch.empty(top_k, dtype=torch.int32, device=dev) if ids is None else ids
    weights = torch.empty(top_k, dtype=torch.float32, device=dev) if weights is None else weights
    fn, args, _keep = _moe_args(x, None, router, shared_gate_row, gate, up, down, shared_gate, shared_up,
                                shared_down, top_k, out, ids, weights, fp16_boundary, stream)
    _check(fn(*args))
    return out, ids, weights


def moe_decode_noalloc(x, router, shared_gate_row, gate: Int4Experts, up: Int4Experts, down: Int4Experts,
                       shared_gate: Int4Weight, shared_up: Int4Weight, shared_down: Int4Weight, top_k: int,
                       out, ids, weights, fp16_boundary=False, stream=None):
    """moe_decode through decodehp_moe_decode_noalloc: the library's fixed per-GPU scratch instead of
    a workspace, so nothing is allocated, here or in the library. The caller passes out fp16 [hidden],
    ids int32 [top_k] and weights fp32 [top_k]; router: bf16 bits (int16) or fp32 [E, hidden].
    Calls that overlap in time on one GPU race on the shared scratch."""
    torch = _torch()
    hidden = gate.cols
    _need(x, torch.float16, "x", hidden)
    _need(shared_gate_row, torch.int16, "shared_gate_row", hidden)
    _need(out, torch.float16, "out", hidden)
    _need(ids, torch.int32, "ids", top_k)
    _need(weights, torch.float32, "weights", top_k)
    rdt = _plain_router(router, gate.count, hidden)
    descs = (gate.desc(), up.desc(), down.desc(), shared_gate.desc(), shared_up.desc(), shared_down.desc())
    _check(lib().decodehp_moe_decode_noalloc(x.data_ptr(), router.data_ptr(), rdt, shared_gate_row.data_ptr(),
                                             *[ctypes.byref(d) for d in descs], top_k,
                                             DHP_MOE_FP16_BOUNDARY if fp16_boundary else 0, out.data_ptr(),
                                             ids.data_ptr(), weights.data_ptr(), _stream(stream)))
    return out, ids, weights


def hc_read(raw, hc_norm, C: int, H: int, down: Int4Weight, up: Int4Weight, inject: Optional[Int4Weight],
            eps: float = 1e-6, mixed=None, inject_w=None, stream=None):
    """One hyper-connection read. raw fp16 [C*H]; hc_norm bf16 bits (int16) [C*H].

    Returns (mixed fp16 [H], inject_w fp32 [C] or None).
    """
    torch = _torch()
    _need(raw, torch.float16, "raw", C * H)
    _need(hc_norm, torch.int16, "hc_norm", C * H)
    dev = raw.device
    mixed = torch.empty(H, dtype=torch.float16, device=dev) if mixed is None else mixed
    _need(mixed, torch.float16, "mixed", H)
    if inject is not None and inject_w is None:
        inject_w = torch.empty(C, dtype=torch.float32, device=dev)
    if inject_w is not None:
        _need(inject_w, torch.float32, "inject_w", C)
    ws = _workspace(workspace_bytes(DHP_OP_HC_READ, C, down.rows), dev, stream=stream)
    dd, ud = down.desc(), up.desc()
    idesc = inject.desc() if inject is not None else None
    _check(lib().decodehp_hc_read(raw.data_ptr(), hc_norm.data_ptr(), C, H, eps, ctypes.byref(dd),
                                  ctypes.byref(ud), ctypes.byref(idesc) if idesc is not None else None,
                                  mixed.data_ptr(), _ptr(inject_w), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)))
    return mixed, (inject_w if inject is not None else None)


def hc_inject(wide, out, inject_w, C: int, H: int, stream=None):
    """wide[c*H + h] += out[h] * inject_w[c] in place (fp16 storage, fp32 math); returns wide."""
    torch = _torch()
    _need(wide, torch.float16, "wide", C * H)
    _need(out, torch.float16, "out", H)
    _need(inject_w, torch.float32, "inject_w", C)
    _check(lib().decodehp_hc_inject(wide.data_ptr(), out.data_ptr(), inject_w.data_ptr(), C, H, _stream(stream)))
    return wide


def _hc_inject_read_args(prev, out, inject_w, hidden, hc_norm, C, H, down, up, inject, mixed, inject_w_next, eps,
                        stream):
    torch = _torch()
    _need(prev, torch.float16, "prev", C * H)
    _need(out, torch.float16, "out", H)
    _need(inject_w, torch.float32, "inject_w", C)
    _need(hidden, torch.float16, "hidden", C * H)
    _need(hc_norm, torch.int16, "hc_norm", C * H)
    _need(mixed, torch.float16, "mixed", H)
    if inject_w_next is not None:
        _need(inject_w_next, torch.float32, "inject_w_next", C)
    ws = _workspace(workspace_bytes(DHP_OP_HC_READ, C, down.rows), prev.device, stream=stream)
    descs = (down.desc(), up.desc(), inject.desc() if inject is not None else None)
    args = (prev.data_ptr(), out.data_ptr(), inject_w.data_ptr(), hidden.data_ptr(), hc_norm.data_ptr(), C, H, eps,
            ctypes.byref(descs[0]), ctypes.byref(descs[1]), ctypes.byref(descs[2]) if descs[2] is not None else None,
            mixed.data_ptr(), _ptr(inject_w_next), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    keep = (descs, prev, out, inject_w, hidden, hc_norm, mixed, inject_w_next, ws, down, up, inject)
    return args, keep


def hc_inject_read(prev, out, inject_w, hc_norm, C: int, H: int, down: Int4Weight, up: Int4Weight,
                   inject: Optional[Int4Weight], hidden=None, mixed=None, inject_w_next=None, eps: float = 1e-6,
                   stream=None):
    """The inject of a sublayer output followed by the next read: hidden = fp16(prev + out * inject_w
    per stream) (prev is not written), then the read of hidden. Returns (hidden fp16 [C*H], mixed fp16 [H],
    inject_w_next fp32 [C] or None)."""
    torch = _torch()
    dev = prev.device
    hidden = torch.empty(C * H, dtype=torch.float16, device=dev) if hidden is None else hidden
    mixed = torch.empty(H, dtype=torch.float16, device=dev) if mixed is None else mixed
    if inject is not None and inject_w_next is None:
        inject_w_next = torch.empty(C, dtype=torch.float32, device=dev)
    args, _keep = _hc_inject_read_args(prev, out, inject_w, hidden, hc_norm, C, H, down, up, inject, mixed,
                                       inject_w_next, eps, stream)
    _check(lib().decodehp_hc_inject_read(*args))
    return hidden, mixed, (inject_w_next if inject is not None else None)


# --------------------------------------------------------------------------- measurement probes

def probe_empty(count: int = 1, stream=None):
    """Launch `count` kernels that do nothing, back to back (the per-launch floor)."""
    _check(lib().decodehp_probe_empty(count, _stream(stream)))


def probe_grid_barrier(blocks: int, n: int, ordered: bool, state, sink, stream=None):
    """One launch of `blocks` blocks passing n grid-wide barriers. state: int32 [4] zeroed device
    tensor (kept between calls); sink: int32 [>= blocks] device tensor (1 per block that never ran
    out of polls)."""
    _check(lib().decodehp_probe_grid_barrier(blocks, n, int(bool(ordered)), state.data_ptr(), sink.data_ptr(),
                                             _stream(stream)))


def probe_read(buf, blocks_per_cu: int = 2, loads_in_flight: int = 4, sink=None, stream=None):
    """Stream the device tensor `buf` once (16-byte nontemporal loads); returns the sink tensor."""
    torch = _torch()
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(16 * 1024, dtype=torch.int32, device=buf.device)
    _check(lib().decodehp_probe_read(buf.data_ptr(), nbytes, blocks_per_cu, loads_in_flight, sink.data_ptr(),
                                     sink.numel(), _stream(stream)))
    return sink


# --------------------------------------------------------------------------- prepared calls

def moe_prefill_workspace_bytes(m: int, n_experts: int, top_k: int, inter: int, hidden: int) -> int:
    return int(lib().decodehp_moe_prefill_workspace_bytes(m, n_experts, top_k, inter, hidden))


def moe_prefill(x, router, shared_gate_row, gate: Int4Experts, up: Int4Experts, down: Int4Experts,
                shared_gate: Int4Weight, shared_up: Int4Weight, shared_down: Int4Weight, top_k: int,
                fp16_boundary=False, out=None, ids=None, weights=None, stream=None):
    """A chunk of m tokens (x fp16 [m, hidden], m <= 128) through the routed MoE layer; row i of
    every output equals moe_decode of x[i], bit for bit.

    Returns (out fp16 [m, hidden], ids int32 [m, top_k], weights fp32 [m, top_k]).
    """
    torch = _torch()
    m, dev = x.shape[0], x.device
    out = torch.empty((m, gate.cols), dtype=torch.float16, device=dev) if out is None else out
    ids = torch.empty((m, top_k), dtype=torch.int32, device=dev) if ids is None else ids
    weights = torch.empty((m, top_k), dtype=torch.float32, device=dev) if weights is None else weights
    fn, args, _keep = _moe_args(x, m, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down,
                                top_k, out, ids, weights, fp16_boundary, stream)
    _check(fn(*args))
    return out, ids, weights


def _hcb_args(raw, hc_norm, C, H, down, up, inject, mixed, inject_w, eps, stream):
    torch = _torch()
    m = raw.shape[0]
    _need(raw, torch.float16, "raw", m * C * H)
    _need(hc_norm, torch.int16, "hc_norm", C * H)
    _need(mixed, torch.float16, "mixed", m * H)
    if inject_w is not None:
        _need(inject_w, torch.float32, "inject_w", m * C)
    ws = _workspace(int(lib().decodehp_hc_read_batched_workspace_bytes(m, C, H, down.rows)), raw.device, "hc_batched", stream=stream)
    descs = (down.desc(), up.desc(), inject.desc() if inject is not None else None)
    args = (raw.data_ptr(), m, hc_norm.data_ptr(), C, H, eps, ctypes.byref(descs[0]), ctypes.byref(descs[1]),
            ctypes.byref(descs[2]) if descs[2] is not None else None, mixed.data_ptr(), _ptr(inject_w), _ptr(ws),
            0 if ws is None else ws.numel(), _stream(stream))
    return args, (descs, raw, hc_norm, mixed, inject_w, ws, down, up, inject)


def hc_read_batched(raw, hc_norm, C: int, H: int, down: Int4Weight, up: Int4Weight, inject: Optional[Int4Weight],
                    eps: float = 1e-6, mixed=None, inject_w=None, stream=None):
    """The read for the m tokens of a chunk: raw fp16 [m, C*H]. Returns (mixed fp16 [m, H],
    inject_w fp32 [m, C] or None)."""
    torch = _torch()
    m, dev = raw.shape[0], raw.device
    mixed = torch.empty((m, H), dtype=torch.float16, device=dev) if mixed is None else mixed
    if inject is not None and inject_w is None:
        inject_w = torch.empty((m, C), dtype=torch.float32, device=dev)
    args, _keep = _hcb_args(raw, hc_norm, C, H, down, up, inject, mixed, inject_w, eps, stream)
    _check(lib().decodehp_hc_read_batched(*args))
    return mixed, (inject_w if inject is not None else None)


def prepare_hc_read_batched(raw, hc_norm, C, H, down, up, inject, mixed, inject_w, eps=1e-6,
                            stream=None) -> "PreparedCall":
    args, keep = _hcb_args(raw, hc_norm, C, H, down, up, inject, mixed, inject_w, eps, stream)
    return PreparedCall(lib().decodehp_hc_read_batched, args, keep)


def hc_inject_batched(wide, out, inject_w, C: int, H: int, stream=None):
    """wide[t, c*H + h] += out[t, h] * inject_w[t, c] in place for the m rows; returns wide."""
    torch = _torch()
    m = wide.shape[0]
    _need(wide, torch.float16, "wide", m * C * H)
    _need(out, torch.float16, "out", m * H)
    _need(inject_w, torch.float32, "inject_w", m * C)
    _check(lib().decodehp_hc_inject_batched(wide.data_ptr(), m, out.data_ptr(), inject_w.data_ptr(), C, H,
                                            _stream(stream)))
    return wide


def prepare_hc_inject_batched(wide, out, inject_w, C, H, stream=None) -> "PreparedCall":
    args = (wide.data_ptr(), wide.shape[0], out.data_ptr(), inject_w.data_ptr(), C, H, _stream(stream))
    return PreparedCall(lib().decodehp_hc_inject_batched, args, (wide, out, inject_w))


class HcBlock:
    """One hyper-connection read's weights: hc_norm bf16 bits (int16 tensor) [C*H], down [R x C*H],
    up [C*H x R], inject [C x C*H] (None for the final mixer)."""

    def __init__(self, hc_norm, down: Int4Weight, up: Int4Weight, inject: Optional[Int4Weight]):
        self.hc_norm, self.down, self.up, self.inject = hc_norm, down, up, inject

    def c(self, keep: list) -> CHcBlock:
        d = [self.down.desc(), self.up.desc(), self.inject.desc() if self.inject is not None else None]
        keep.extend(d)
        return CHcBlock(self.hc_norm.data_ptr(), ctypes.pointer(d[0]), ctypes.pointer(d[1]),
                        ctypes.pointer(d[2]) if d[2] is not None else None)


class DecodeLayer:
    """Weights of one decoder layer: the attn and mlp hyper-connection reads, the INT4 [H x H]
    stand-in for the attention sublayer, and the MoE (as moe_decode takes them)."""

    def __init__(self, attn_hc: HcBlock, sublayer: Int4Weight, mlp_hc: HcBlock, router, shared_gate_row,
                 gate: Int4Experts, up: Int4Experts, down: Int4Experts, shared_gate: Int4Weight,
                 shared_up: Int4Weight, shared_down: Int4Weight, top_k: int, fp16_boundary: bool = False):
        self.__dict__.update(locals())
        del self.__dict__["self"]

    def c(self, keep: list) -> CDecodeLayer:
        torch = _torch()
        e = [self.gate.desc(), self.up.desc(), self.down.desc()]
        w = [self.sublayer.desc(), self.shared_gate.desc(), self.shared_up.desc(), self.shared_down.desc()]
        keep.extend(e + w)
        return CDecodeLayer(self.attn_hc.c(keep), ctypes.pointer(w[0]), self.mlp_hc.c(keep), self.router.data_ptr(),
                            DHP_BF16 if self.router.dtype == torch.int16 else DHP_F32, self.shared_gate_row.data_ptr(),
                            ctypes.pointer(e[0]), ctypes.pointer(e[1]), ctypes.pointer(e[2]), ctypes.pointer(w[1]),
                            ctypes.pointer(w[2]), ctypes.pointer(w[3]), self.top_k,
                            DHP_MOE_FP16_BOUNDARY if self.fp16_boundary else 0)


def _layer_args(x, C, H, layers, mixer, hidden, mixed_out, eps, stream=None, private_ws=False):
    torch = _torch()
    _need(x, torch.float16, "x", H)
    _need(hidden, torch.float16, "hidden", C * H)
    _need(mixed_out, torch.float16, "mixed_out", H)
    keep = []
    arr = (CDecodeLayer * max(1, len(layers)))(*[L.c(keep) for L in layers])
    mix = mixer.c(keep)
    nbytes = int(lib().decodehp_decode_layers_workspace_bytes(C, H, arr, len(layers), ctypes.byref(mix)))
    if nbytes == 0:
        raise DecodeHPError(-1, "null or inconsistent layer descriptors")
    if private_ws:     # a captured graph pins its workspace for its lifetime: never shared
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    else:
        ws = _workspace(nbytes, x.device, "layers", stream=stream)
    keep.extend([arr, mix, ws, layers, mixer, x, hidden, mixed_out])
    return (x.data_ptr(), C, H, eps, arr, len(layers), ctypes.byref(mix), hidden.data_ptr(), mixed_out.data_ptr(),
            ws.data_ptr(), ws.numel()), keep


def decode_layers(x, C: int, H: int, layers, mixer: HcBlock, hidden=None, mixed_out=None, eps=1e-6, stream=None):
    """One token (x fp16 [H]) through the layers and the final mixer, as a launch sequence.
    Returns (hidden fp16 [C*H] after the last layer, mixed fp16 [H] from the mixer)."""
    torch = _torch()
    hidden = torch.empty(C * H, dtype=torch.float16, device=x.device) if hidden is None else hidden
    mixed_out = torch.empty(H, dtype=torch.float16, device=x.device) if mixed_out is None else mixed_out
    args, _keep = _layer_args(x, C, H, layers, mixer, hidden, mixed_out, eps, stream=stream)
    _check(lib().decodehp_decode_layers(*args, _stream(stream)))
    return hidden, mixed_out


def prepare_decode_layers(x, C: int, H: int, layers, mixer: HcBlock, hidden, mixed_out, eps=1e-6,
                          stream=None) -> PreparedCall:
    args, keep = _layer_args(x, C, H, layers, mixer, hidden, mixed_out, eps, stream=stream)
    return PreparedCall(lib().decodehp_decode_layers, (*args, _stream(stream)), keep)


class LayerGraph:
    """The decode_layers sequence captured once as a HIP graph over fixed buffers (x, hidden,
    mixed_out and a workspace). Capture runs the sequence once. launch() replays it on a stream;
    write the next token into x first."""

    def __init__(self, x, C: int, H: int, layers, mixer: HcBlock, hidden, mixed_out, eps=1e-6):
        args, self._keep = _layer_args(x, C, H, layers, mixer, hidden, mixed_out, eps, private_ws=True)
        self._g = ctypes.c_void_p()
        _check(lib().decodehp_graph_capture_decode_layers(*args, ctypes.byref(self._g)))
        self.x, self.hidden, self.mixed = x, hidden, mixed_out

    def launch(self, stream=None):
        rc = lib().decodehp_graph_launch(self._g, _stream(stream))
        if rc != 0:
            _check(rc)

    def __del__(self):
        if getattr(self, "_g", None) and self._g.value and _lib is not None:
            _lib.decodehp_graph_destroy(self._g)
            self._g = ctypes.c_void_p()


class PreparedCall:
    """One entry-point call with every argument marshalled up front; calling it only crosses
    the C boundary (for launch loops where per-call Python work would starve the GPU).
    Holds references to every tensor and descriptor it points at."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc)


def prepare_gemv(w: Int4Weight, x, y, argmax=None, stream=None, matrix_cores=False) -> PreparedCall:
    torch = _torch()
    x2 = x.reshape(-1, w.cols)
    m = x2.shape[0]
    _need(x2, torch.float16, "x")
    _need(y, y.dtype, "y", m * w.rows)
    ws = _workspace(workspace_bytes(DHP_OP_GEMV_ARGMAX, w.rows, m), x.device, "argmax", stream=stream) if argmax is not None else None
    d = w.desc()
    args = (ctypes.byref(d), x2.data_ptr(), m, y.data_ptr(), DHP_F32 if y.dtype == torch.float32 else DHP_F16,
            _ptr(argmax), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    fn = lib().decodehp_dequant_gemv_mc if matrix_cores else lib().decodehp_dequant_gemv
    return PreparedCall(fn, args, (d, x2, y, argmax, ws, w))


def prepare_gemm_batched(w: Int4Weight, x, y, stream=None) -> PreparedCall:
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(y, torch.float16, "y", x.shape[0] * w.rows)
    d = w.desc()
    args = (ctypes.byref(d), x.data_ptr(), x.shape[0], y.data_ptr(), _stream(stream))
    return PreparedCall(lib().decodehp_dequant_gemm_batched, args, (d, x, y, w))


def prepare_moe(x, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k, out, ids,
                weights, fp16_boundary=False, stream=None) -> PreparedCall:
    fn, args, keep = _moe_args(x, None, router, shared_gate_row, gate, up, down, shared_gate, shared_up,
                               shared_down, top_k, out, ids, weights, fp16_boundary, stream)
    return PreparedCall(fn, args, keep)


def prepare_moe_prefill(x, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k, out,
                        ids, weights, fp16_boundary=False, stream=None) -> PreparedCall:
    fn, args, keep = _moe_args(x, x.shape[0], router, shared_gate_row, gate, up, down, shared_gate, shared_up,
                               shared_down, top_k, out, ids, weights, fp16_boundary, stream)
    return PreparedCall(fn, args, keep)


def prepare_hc_read(raw, hc_norm, C, H, down, up, inject, mixed, inject_w, eps=1e-6, stream=None) -> PreparedCall:
    ws = _workspace(workspace_bytes(DHP_OP_HC_READ, C, down.rows), raw.device, stream=stream)
    descs = (down.desc(), up.desc(), inject.desc() if inject is not None else None)
    args = (raw.data_ptr(), hc_norm.data_ptr(), C, H, eps, ctypes.byref(descs[0]), ctypes.byref(descs[1]),
            ctypes.byref(descs[2]) if descs[2] is not None else None, mixed.data_ptr(), _ptr(inject_w), _ptr(ws),
            0 if ws is None else ws.numel(), _stream(stream))
    return PreparedCall(lib().decodehp_hc_read, args, (descs, raw, hc_norm, mixed, inject_w, ws, down, up, inject))


def prepare_hc_inject(wide, out, inject_w, C, H, stream=None) -> PreparedCall:
    args = (wide.data_ptr(), out.data_ptr(), inject_w.data_ptr(), C, H, _stream(stream))
    return PreparedCall(lib().decodehp_hc_inject, args, (wide, out, inject_w))


def prepare_hc_inject_read(prev, out, inject_w, hidden, hc_norm, C, H, down, up, inject, mixed, inject_w_next,
                           eps=1e-6, stream=None) -> PreparedCall:
    args, keep = _hc_inject_read_args(prev, out, inject_w, hidden, hc_norm, C, H, down, up, inject, mixed,
                                      inject_w_next, eps, stream)
    return PreparedCall(lib().decodehp_hc_inject_read, args, keep)
