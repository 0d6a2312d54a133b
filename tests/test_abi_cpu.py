"""The C ABI on the host: the library loads, exports every declared symbol, and rejects
bad arguments with the documented codes before touching a device."""
import ctypes
import os
import re

import pytest

import hyper_connections_amd as hca
from helpers import gpu_present

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decodehp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hca.LIB_PATH), reason="libdecodehp.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(decodehp_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("decodehp_dequant_gemv", "decodehp_dequant_gemm_batched", "decodehp_moe_decode",
              "decodehp_moe_prefill", "decodehp_moe_prefill_workspace_bytes",
              "decodehp_hc_read", "decodehp_hc_inject", "decodehp_workspace_bytes", "decodehp_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(hca.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_version():
    assert hca.lib().decodehp_version() >= 1


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def int4(codes=FAKE, scales=FAKE, biases=FAKE, rows=16, cols=128, group=64):
    return hca.CInt4(codes, scales, biases, rows, cols, group)


def gemv(w, x=FAKE, m=1, y=FAKE, dt=0, am=None, ws=None, wsb=0):
    L = hca.lib()
    return L.decodehp_dequant_gemv(ctypes.byref(w) if w is not None else None, x, m, y, dt, am, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(codes=0), -1), (dict(scales=0), -1), (dict(rows=0), -1), (dict(cols=-64), -1),
    (dict(cols=96), -2), (dict(group=32), -2), (dict(cols=16448), -2),
    (dict(codes=FAKE + 8), -3), (dict(scales=FAKE + 1), -3),
])
def test_gemv_rejects_bad_weights(kw, code):
    assert gemv(int4(**kw)) == code
    assert hca.lib().decodehp_last_error().decode()


def test_gemv_rejects_bad_calls():
    assert gemv(None) == -1
    assert gemv(int4(), x=0) == -1
    assert gemv(int4(), m=0) == -2
    assert gemv(int4(), m=17) == -2
    assert gemv(int4(), dt=2) == -2
    assert gemv(int4(), x=FAKE + 2) == -3
    assert gemv(int4(), y=FAKE + 1) == -3
    assert gemv(int4(), am=FAKE, ws=None) == -4
    need = hca.workspace_bytes(hca.DHP_OP_GEMV_ARGMAX, 16, 1)
    assert need > 0
    assert gemv(int4(), am=FAKE, ws=FAKE, wsb=need - 1) == -4


def test_gemm_batched_rejects_bad_calls():
    L = hca.lib()
    f = lambda w, m=128, x=FAKE, y=FAKE: L.decodehp_dequant_gemm_batched(ctypes.byref(w), x, m, y, None)
    assert f(int4(), m=0) == -2
    assert f(int4(), m=129) == -2
    assert f(int4(rows=24)) == -2
    assert f(int4(), x=FAKE + 4) == -3
    assert f(int4(cols=100)) == -2


def test_error_message_is_per_call():
    assert gemv(int4(group=32)) == -2
    assert "group" in hca.lib().decodehp_last_error().decode()


@pytest.mark.skipif(gpu_present(), reason="a GPU is visible; a valid call would launch")
def test_valid_call_without_device_reports_no_device():
    assert gemv(int4()) == -5
    assert "device" in hca.lib().decodehp_last_error().decode()


def test_pack_int4_codes_layout():
    import numpy as np
    q = np.array([[1, 2, 3, 4, 15, 0, 7, 8]], np.uint8)
    p = hca.pack_int4_codes(q)
    assert p.tolist() == [[0x21, 0x43, 0x0F, 0x87]]
    with pytest.raises(ValueError):
        hca.pack_int4_codes(np.array([[16, 0]], np.uint8))


def experts(count=8, rows=64, cols=512, **kw):
    return hca.CInt4Experts(int4(rows=rows, cols=cols, **kw), rows * cols // 2, 2 * rows * (cols // 64), count)


def moe(top_k=2, flags=0, rdt=2, E=8, hidden=512, inter=64, ws=FAKE, wsb=1 << 20, x=FAKE, down_rows=None,
        sh_rows=None):
    L = hca.lib()
    g, u = experts(E, inter, hidden), experts(E, inter, hidden)
    d = experts(E, down_rows or hidden, inter)
    sg, su = int4(rows=sh_rows or inter, cols=hidden), int4(rows=inter, cols=hidden)
    sd = int4(rows=hidden, cols=inter)
    return L.decodehp_moe_decode(x, FAKE, rdt, FAKE, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                 ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), top_k, flags, FAKE,
                                 FAKE, FAKE, ws, wsb, None)


def test_moe_rejects_bad_calls():
    assert moe(x=0) == -1
    assert moe(top_k=0) == -2
    assert moe(top_k=11) == -2                 # at most DHP_MOE_MAX_TOP_K = 10 slots
    assert moe(top_k=8, E=4) == -2
    assert moe(rdt=0) == -2
    assert moe(flags=2) == -2
    assert moe(hidden=640) == -2               # hidden % 512
    assert moe(inter=2048) == -2
    assert moe(E=2048) == -2
    assert moe(down_rows=256) == -1            # down must be [hidden x inter]
    assert moe(sh_rows=128) == -1
    assert moe(x=FAKE + 4) == -3
    assert moe(ws=None) == -4
    need = hca.workspace_bytes(hca.DHP_OP_MOE_DECODE, 8, 2, 64)
    assert need >= (8 + 3 * 64) * 4
    assert moe(wsb=need - 1) == -4


def moe_ex(router=True, rdt=3, weights=FAKE, elem=None, escale=None, top_k=2, E=12, prefill=False):
    L = hca.lib()
    hidden, inter = 512, 64
    g, u = experts(E, inter, hidden), experts(E, inter, hidden)
    d = experts(E, hidden, inter)
    sg, su, sd = int4(rows=inter, cols=hidden), int4(rows=inter, cols=hidden), int4(rows=hidden, cols=inter)
    r = hca.CRouter(weights, rdt, elem, escale)
    rp = ctypes.byref(r) if router else None
    tail = (FAKE, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ctypes.byref(sg), ctypes.byref(su),
            ctypes.byref(sd), top_k, 0, FAKE, FAKE, FAKE, FAKE, 1 << 24, None)
    if prefill:
        return L.decodehp_moe_prefill_ex(FAKE, 4, rp, *tail)
    return L.decodehp_moe_decode_ex(FAKE, rp, *tail)


@pytest.mark.parametrize("prefill", [False, True])
def test_moe_ex_rejects_bad_routers(prefill):
    assert moe_ex(router=False, prefill=prefill) == -1
    assert moe_ex(weights=0, prefill=prefill) == -1
    assert moe_ex(rdt=4, prefill=prefill) == -2
    assert moe_ex(rdt=0, prefill=prefill) == -2            # fp16 routers are not a variant
    assert moe_ex(weights=FAKE + 4, prefill=prefill) == -3  # int8 rows need 8-byte alignment
    assert moe_ex(rdt=2, weights=FAKE + 8, prefill=prefill) == -3
    assert moe_ex(elem=FAKE + 8, prefill=prefill) == -3
    assert moe_ex(escale=FAKE + 2, prefill=prefill) == -3
    assert moe_ex(top_k=11, prefill=prefill) == -2
    assert moe_ex(top_k=11, E=10, prefill=prefill) == -2


@pytest.mark.skipif(gpu_present(), reason="checks the no-device path")
@pytest.mark.parametrize("prefill", [False, True])
def test_moe_ex_valid_calls_reach_the_device_check(prefill):
    assert moe_ex(weights=FAKE + 8, elem=FAKE, escale=FAKE + 4, top_k=10, prefill=prefill) == -5
    assert moe_ex(rdt=1, top_k=10, E=10, prefill=prefill) == -5
    assert moe(top_k=10, E=10) == -5


def moe_prefill(m=4, top_k=2, flags=0, E=8, hidden=512, inter=64, ws=FAKE, wsb=1 << 24, x=FAKE, ids=FAKE):
    L = hca.lib()
    g, u = experts(E, inter, hidden), experts(E, inter, hidden)
    d = experts(E, hidden, inter)
    sg, su, sd = int4(rows=inter, cols=hidden), int4(rows=inter, cols=hidden), int4(rows=hidden, cols=inter)
    return L.decodehp_moe_prefill(x, m, FAKE, 2, FAKE, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                  ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), top_k, flags, FAKE,
                                  ids, FAKE, ws, wsb, None)


def test_moe_prefill_rejects_bad_calls():
    assert moe_prefill(m=0) == -2
    assert moe_prefill(m=129) == -2
    assert moe_prefill(ids=0) == -1
    assert moe_prefill(top_k=11) == -2
    assert moe_prefill(flags=4) == -2
    assert moe_prefill(hidden=640) == -2
    assert moe_prefill(x=FAKE + 4) == -3
    assert moe_prefill(ws=None) == -4
    need = hca.moe_prefill_workspace_bytes(4, 8, 2, 64, 512)
    # logits [4][8], gate logits [4], act [4][3][64] and slot dots [4][3][512], fp32
    assert need >= (4 * 8 + 4 + 4 * 3 * 64 + 4 * 3 * 512) * 4
    assert moe_prefill(wsb=need - 1) == -4
    assert hca.moe_prefill_workspace_bytes(0, 8, 2, 64, 512) == 0
    assert hca.moe_prefill_workspace_bytes(129, 8, 2, 64, 512) == 0


def hc_read(C=4, H=512, R=64, inject=True, iw=FAKE, ws=FAKE, wsb=1 << 16, eps=1e-6, raw=FAKE, up_cols=None):
    L = hca.lib()
    down, up = int4(rows=R, cols=C * H), int4(rows=C * H, cols=up_cols or R)
    inj = int4(rows=C, cols=C * H)
    return L.decodehp_hc_read(raw, FAKE, C, H, eps, ctypes.byref(down), ctypes.byref(up),
                              ctypes.byref(inj) if inject else None, FAKE, iw, ws, wsb, None)


def test_hc_read_rejects_bad_calls():
    assert hc_read(raw=0) == -1
    assert hc_read(C=3) == -2                  # not a power of two
    assert hc_read(C=32) == -2
    assert hc_read(H=96) == -2
    assert hc_read(C=1, H=1024) == -2          # C*H not a multiple of 2048
    assert hc_read(R=96) == -2
    assert hc_read(up_cols=128) == -1
    assert hc_read(inject=False) == -1         # inject_w without inject
    assert hc_read(iw=None) == -1              # inject without inject_w
    assert hc_read(eps=-1.0) == -1
    assert hc_read(raw=FAKE + 8) == -3
    assert hc_read(ws=None) == -4
    assert hc_read(wsb=hca.workspace_bytes(hca.DHP_OP_HC_READ, 4, 64) - 1) == -4


def test_hc_inject_rejects_bad_calls():
    L = hca.lib()
    f = lambda wide=FAKE, C=4, H=64, out=FAKE: L.decodehp_hc_inject(wide, out, FAKE, C, H, None)
    assert f(wide=0) == -1
    assert f(C=0) == -1
    assert f(C=17) == -2
    assert f(H=12) == -2
    assert f(out=FAKE + 2) == -3


def _layer_descs(E=8, C=4, H=512, R=64, inter=64, mixer_inject=False):
    hb = lambda inj: hca.CHcBlock(FAKE, ctypes.pointer(int4(rows=R, cols=C * H)), ctypes.pointer(int4(rows=C * H, cols=R)),
                                  ctypes.pointer(int4(rows=C, cols=C * H)) if inj else None)
    L = hca.CDecodeLayer(hb(True), ctypes.pointer(int4(rows=H, cols=H)), hb(True), FAKE, 2, FAKE,
                         ctypes.pointer(experts(E, inter, H)), ctypes.pointer(experts(E, inter, H)),
                         ctypes.pointer(experts(E, H, inter)), ctypes.pointer(int4(rows=inter, cols=H)),
                         ctypes.pointer(int4(rows=inter, cols=H)), ctypes.pointer(int4(rows=H, cols=inter)), 2, 0)
    return (hca.CDecodeLayer * 1)(L), hb(mixer_inject)


def test_decode_layers_rejects_bad_calls():
    L = hca.lib()
    layers, mixer = _layer_descs()
    need = L.decodehp_decode_layers_workspace_bytes(4, 512, layers, 1, ctypes.byref(mixer))
    assert need >= 2 * 512 * 2 + 4 * 4
    _, bad_mixer = _layer_descs(mixer_inject=True)                 # the final mixer has no inject
    assert L.decodehp_decode_layers_workspace_bytes(4, 512, layers, 1, ctypes.byref(bad_mixer)) == 0
    assert L.decodehp_decode_layers(None, 4, 512, 1e-6, layers, 1, ctypes.byref(mixer), FAKE, FAKE, FAKE, need,
                                    None) == -1
    assert L.decodehp_decode_layers(FAKE, 4, 512, 1e-6, layers, 1, ctypes.byref(mixer), FAKE, FAKE, FAKE, need - 1,
                                    None) == -4
    assert L.decodehp_decode_layers(FAKE + 8, 4, 512, 1e-6, layers, 1, ctypes.byref(mixer), FAKE, FAKE, FAKE, need,
                                    None) == -3
    assert L.decodehp_graph_capture_decode_layers(FAKE, 4, 512, 1e-6, layers, 1, ctypes.byref(mixer), FAKE, FAKE,
                                                  FAKE, need, None) == -1
    assert L.decodehp_graph_launch(None, None) == -1
    L.decodehp_graph_destroy(None)


def test_hc_batched_rejects_bad_calls():
    L = hca.lib()
    C, H, R = 4, 512, 64
    down, up, inj = int4(rows=R, cols=C * H), int4(rows=C * H, cols=R), int4(rows=C, cols=C * H)
    need = L.decodehp_hc_read_batched_workspace_bytes(8, C, H, R)
    assert need >= 8 * C * H * (2 + 4)                      # normed fp16 and the up output fp32
    assert L.decodehp_hc_read_batched_workspace_bytes(0, C, H, R) == 0
    f = lambda m=8, iw=FAKE, ws=FAKE, wsb=need, mixed=FAKE: L.decodehp_hc_read_batched(
        FAKE, m, FAKE, C, H, 1e-6, ctypes.byref(down), ctypes.byref(up), ctypes.byref(inj), mixed, iw, ws, wsb, None)
    assert f(m=0) == -2 and f(m=129) == -2
    assert f(iw=None) == -1
    assert f(mixed=FAKE + 8) == -3
    assert f(wsb=need - 1) == -4
    g = lambda m=8, wide=FAKE: L.decodehp_hc_inject_batched(wide, m, FAKE, FAKE, C, H, None)
    assert g(m=0) == -2 and g(wide=None) == -1 and g(wide=FAKE + 8) == -3


def test_probe_grid_barrier_rejects_bad_calls():
    L = hca.lib()
    assert L.decodehp_probe_grid_barrier(64, 1, 1, None, FAKE, None) == -1
    assert L.decodehp_probe_grid_barrier(64, 1, 1, FAKE, None, None) == -1
    assert L.decodehp_probe_grid_barrier(64, -1, 1, FAKE, FAKE, None) == -2
    assert L.decodehp_probe_grid_barrier(64, 10001, 0, FAKE, FAKE, None) == -2


def test_probe_read_rejects_bad_calls():
    L = hca.lib()
    assert L.decodehp_probe_read(0, 1 << 20, 2, 4, FAKE, 4096, None) == -1
    assert L.decodehp_probe_read(FAKE, 0, 2, 4, FAKE, 4096, None) == -1
    assert L.decodehp_probe_read(FAKE, (1 << 20) + 8, 2, 4, FAKE, 4096, None) == -3
    assert L.decodehp_probe_read(FAKE + 8, 1 << 20, 2, 4, FAKE, 4096, None) == -3
    assert L.decodehp_probe_read(FAKE, 1 << 20, 0, 4, FAKE, 4096, None) == -2
    assert L.decodehp_probe_read(FAKE, 1 << 20, 17, 4, FAKE, 4096, None) == -2
    assert L.decodehp_probe_read(FAKE, 1 << 20, 2, 3, FAKE, 4096, None) == -2


def moe_noalloc(top_k=2, E=8, hidden=512, inter=64, x=FAKE):
    L = hca.lib()
    g, u = experts(E, inter, hidden), experts(E, inter, hidden)
    d = experts(E, hidden, inter)
    sg, su, sd = int4(rows=inter, cols=hidden), int4(rows=inter, cols=hidden), int4(rows=hidden, cols=inter)
    return L.decodehp_moe_decode_noalloc(x, FAKE, 2, FAKE, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                         ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), top_k, 0, FAKE,
                                         FAKE, FAKE, None)


def test_moe_noalloc_checks_and_scratch_limit():
    # the checks of decodehp_moe_decode, then the fixed scratch's limit, both before any device call
    assert moe_noalloc(x=0) == -1
    assert moe_noalloc(top_k=11) == -2
    assert moe_noalloc(E=1024, inter=1024, top_k=10) == -4      # 58,624 bytes > 48 KiB
    assert "scratch" in hca.lib().decodehp_last_error().decode()
    assert hca.workspace_bytes(hca.DHP_OP_MOE_DECODE, 1024, 10, 640) <= 49152
    assert moe_noalloc(E=1024, inter=640, top_k=10) == -5       # fits; no device here
    assert moe_noalloc(E=256, inter=512, top_k=8) == -5


def test_hc_inject_read_rejects_overlaps_and_bad_calls():
    L = hca.lib()
    C, H, R = 4, 512, 64
    down, up, inj = int4(rows=R, cols=C * H), int4(rows=C * H, cols=R), int4(rows=C, cols=C * H)
    P, O, W, HID, W2 = FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20), FAKE + (4 << 20)

    def f(prev=P, out=O, iw=W, hidden=HID, iw_next=W2, ws=FAKE + (5 << 20), wsb=1 << 16, C=C):
        return L.decodehp_hc_inject_read(prev, out, iw, hidden, FAKE, C, H, 1e-6, ctypes.byref(down),
                                         ctypes.byref(up), ctypes.byref(inj), FAKE, iw_next, ws, wsb, None)
    assert f() == -5                                # valid; no device here
    assert f(prev=0) == -1
    assert f(hidden=P + 4096 - 16) == -1            # overlaps prev (C*H*2 = 4096 bytes)
    assert f(hidden=P + 4096) == -5                 # just past it
    assert f(hidden=O) == -1                        # overlaps out
    assert f(iw_next=W + 8) == -1                   # overlaps the consumed gates
    assert f(iw_next=W + 16) == -5
    assert f(C=3) == -2
    assert f(hidden=HID + 8) == -3
    assert f(ws=None) == -4


def test_gemv_mc_checks_like_gemv():
    L = hca.lib()
    w = int4(rows=64, cols=512)
    for fn in (L.decodehp_dequant_gemv, L.decodehp_dequant_gemv_mc):
        assert fn(ctypes.byref(w), 0, 2, FAKE, 1, None, None, 0, None) == -1
        assert fn(ctypes.byref(w), FAKE, 17, FAKE, 1, None, None, 0, None) == -2
        assert fn(ctypes.byref(w), FAKE + 8, 2, FAKE, 1, None, None, 0, None) == -3
        assert fn(ctypes.byref(w), FAKE, 2, FAKE, 1, FAKE, None, 0, None) == -4
        assert fn(ctypes.byref(w), FAKE, 2, FAKE, 1, None, None, 0, None) == -5
