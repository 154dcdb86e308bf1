"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/mok.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mok.h")


@pytest.fixture(scope="module")
def mok():
    from mixture_experts_layer_stable_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from mixture_experts_layer_stable_amd import mok as m
    return m


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mok_status|const char\*|int32_t)\s+(mok_\w+)\s*\(", src, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("mok_route", "mok_schedule_build", "mok_moe_forward", "mok_moe_backward", "mok_workspace_query"):
        assert n in names


def test_library_exports_every_declared_symbol(mok):
    lib = ctypes.CDLL(mok.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(mok.EXPORTS)
    assert mok.version() == 301


def test_status_strings(mok):
    for st in range(8):
        assert mok._lib.mok_status_string(st)
    assert mok._lib.mok_status_string(6) != mok._lib.mok_status_string(99)
    assert mok._lib.mok_status_string(7) != mok._lib.mok_status_string(99)


def _d(mok, **kw):
    base = dict(T=64, H=128, E=8, k=2, I=256, act=mok.BF16)
    base.update(kw)
    return mok.Desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), 3), (dict(k=9), 3), (dict(E=0), 3), (dict(E=1025), 3), (dict(k=17, E=32), 3),
    (dict(H=100), 3), (dict(I=96), 3), (dict(T=-1), 3), (dict(tile_m=48), 3), (dict(grid=-2), 3),
    (dict(act=2), 4), (dict(act=0, gemm=2), 4), (dict(T=1 << 29, k=8), 3),
    (dict(flags=2), 4), (dict(mb_count=2), 3), (dict(gemm=2, mb_count=2, mb_index=2), 3),
    (dict(gemm=2, mb_index=-1), 3), (dict(gemm=2, mb_count=-1), 3), (dict(gemm=2, ring=-1), 3),
    (dict(gemm=2, T=1 << 20, H=4096, E=8, k=8, mb_count=64), 3),
    (dict(gemm=3, H=128), 3), (dict(gemm=3, H=256, I=128), 3), (dict(act=0, gemm=3, H=256), 4),
    (dict(gemm=4), 4),
])
def test_descriptor_validation(mok, kw, status):
    with pytest.raises(mok.MokError) as ei:
        mok.workspace_query(_d(mok, **kw))
    assert ei.value.status == status


def test_workspace_sizes_cover_worst_case(mok):
    d = _d(mok, T=2048, H=1024, E=32, k=2, I=512)
    s = mok.workspace_query(d)
    R = d.R
    assert s["sched"] >= 4 * (2 * R + 2 * d.E) + 16 * (R // 32 + d.E)
    assert s["saved"] >= 2 * R * 3 * d.I
    assert s["fwd_ws"] >= 2 * R * d.H
    assert s["bwd_ws"] >= 2 * R * (2 * d.I + d.H) + 4 * R
    lay = mok.saved_layout_query(d)
    assert lay["h_offset"] >= 2 * R * 2 * d.I and lay["h_offset"] % 256 == 0


def test_mxfp8_workspace_sizes(mok):
    """MXFP8: ring slots of quantised rows and partials, the stash of every micro-batch,
    and the token-axis operands padded to 128 rows per expert."""
    for M, S in ((1, 1), (8, 2)):
        d = _d(mok, T=256, H=256, E=8, k=2, I=128, gemm=mok.MXFP8, mb_count=M, ring=S)
        s = mok.workspace_query(d)
        R = d.R
        assert s["fwd_ws"] >= S * (d.T * d.H * 33 // 32 + R * d.I * 33 // 32 + 2 * R * d.H)
        stash = M * R * (2 * d.H + 2 * d.H + 2 * d.I + 4 * d.I + 8)
        kmax = M * R + 128 * d.E
        flush = kmax * (2 * d.H + d.I + 2 * d.I) * 33 // 32 + 4 * kmax
        assert s["bwd_ws"] >= S * (d.T * d.H + R * 2 * d.I + 2 * R * d.H) + stash + flush
        assert s["saved"] == mok.workspace_query(_d(mok, T=256, H=256, E=8, k=2, I=128))["saved"]


def test_mxfp4_workspace_sizes(mok):
    """MXFP4: quantised rows hold two E2M1 codes per byte (scales as for MXFP8), and the
    token-axis operands are padded to 256 rows per expert."""
    for M, S in ((1, 1), (8, 2)):
        d4 = _d(mok, T=256, H=256, E=8, k=2, I=256, gemm=mok.MXFP4, mb_count=M, ring=S)
        d8 = _d(mok, T=256, H=256, E=8, k=2, I=256, gemm=mok.MXFP8, mb_count=M, ring=S)
        s4, s8 = mok.workspace_query(d4), mok.workspace_query(d8)
        R = d4.R
        assert s4["fwd_ws"] >= S * (d4.T * d4.H * 17 // 32 + R * d4.I * 17 // 32 + 2 * R * d4.H)
        assert s4["fwd_ws"] < s8["fwd_ws"]
        kmax = M * R + 256 * d4.E
        flush = kmax * (2 * d4.H + d4.I + 2 * d4.I) * 17 // 32 + 4 * kmax
        stash = M * R * (2 * d4.H + 2 * d4.H + 2 * d4.I + 4 * d4.I + 8)
        assert s4["bwd_ws"] >= S * (d4.T * d4.H // 2 + R * d4.I + 2 * R * d4.H) + stash + flush
        assert s4["saved"] == s8["saved"]


def test_null_and_alignment_rejected_before_launch(mok):
    d = _d(mok)
    lib = mok._lib
    c = d.c()
    # x = NULL
    st = lib.mok_route(ctypes.byref(c), None, ctypes.c_void_p(4096), None, ctypes.c_void_p(4096),
                       ctypes.c_void_p(4096), None, None)
    assert st == 1
    # misaligned idx
    st = lib.mok_route(ctypes.byref(c), ctypes.c_void_p(4096), ctypes.c_void_p(4096), None, ctypes.c_void_p(4100),
                       ctypes.c_void_p(4096), None, None)
    assert st == 2
    # NULL schedule / weights struct
    st = lib.mok_schedule_build(ctypes.byref(c), ctypes.c_void_p(4096), None, 1 << 30, None)
    assert st == 1
    st = lib.mok_moe_forward(ctypes.byref(c), ctypes.c_void_p(4096), None, None, None, None, None, 0, None, 0, None)
    assert st == 1
    # MXFP8: weights_quantize needs gemm = MXFP8 and every output pointer
    q = mok._MxWeights(*([4096] * 8))
    st = lib.mok_weights_quantize(ctypes.byref(c), ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.byref(q),
                                  None)
    assert st == 4
    cm = _d(mok, gemm=mok.MXFP8).c()
    q.w1ts = None
    st = lib.mok_weights_quantize(ctypes.byref(cm), ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.byref(q),
                                  None)
    assert st == 1
    q.w1ts = 4100
    st = lib.mok_weights_quantize(ctypes.byref(cm), ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.byref(q),
                                  None)
    assert st == 2
    # MXFP8 forward without the quantised weights
    w = mok._Weights(4096, 4096, None)
    big = 1 << 40
    st = lib.mok_moe_forward(ctypes.byref(cm), ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                             ctypes.byref(w), ctypes.c_void_p(4096), ctypes.c_void_p(4096), big, ctypes.c_void_p(4096),
                             big, None)
    assert st in (1, 5)


def test_undersized_buffers_rejected_before_launch(mok):
    """Each caller buffer is compared with mok_workspace_query's size before the device is
    touched: one byte short gives MOK_ERR_WORKSPACE (no GPU needed), enough gives another
    status (here MOK_ERR_HIP or a later check, since there is no device)."""
    lib = mok._lib
    P = ctypes.c_void_p
    for kw in (dict(), dict(gemm=mok.MXFP8, mb_count=4, ring=2), dict(act=mok.F32)):
        d = _d(mok, T=256, H=256, E=8, k=2, I=128, **kw)
        c = d.c()
        s = mok.workspace_query(d)
        w = mok._Weights(4096, 4096, None)
        st = lib.mok_schedule_build(ctypes.byref(c), P(4096), P(4096), s["sched"] - 1, None)
        assert st == mok.ERR_WORKSPACE
        st = lib.mok_schedule_build(ctypes.byref(c), P(4096), P(4096), s["sched"], None)
        assert st != mok.ERR_WORKSPACE
        for saved, ws in ((s["saved"] - 1, s["fwd_ws"]), (s["saved"], s["fwd_ws"] - 1)):
            st = lib.mok_moe_forward(ctypes.byref(c), P(4096), P(4096), P(4096), ctypes.byref(w), P(4096), P(4096),
                                     saved, P(4096), ws, None)
            assert st == mok.ERR_WORKSPACE, (kw, saved, ws)
        st = lib.mok_moe_forward(ctypes.byref(c), P(4096), P(4096), P(4096), ctypes.byref(w), P(4096), P(4096),
                                 s["saved"], P(4096), s["fwd_ws"], None)
        assert st != mok.ERR_WORKSPACE
        for saved, ws in ((s["saved"] - 1, s["bwd_ws"]), (s["saved"], s["bwd_ws"] - 1)):
            st = lib.mok_moe_backward(ctypes.byref(c), P(4096), P(4096), P(4096), P(4096), ctypes.byref(w), None,
                                      P(4096), saved, P(4096), P(4096), P(4096), P(4096), P(4096), None, P(4096), ws,
                                      None)
            assert st == mok.ERR_WORKSPACE, (kw, saved, ws)


def test_trace_binding_checks(mok):
    """mok_trace_bind validates the caller-owned trace and unbinds with NULL."""
    lib = mok._lib
    t = mok._Trace()
    assert lib.mok_trace_bind(ctypes.byref(t)) == 1          # NULL filter / events
    ev = (ctypes.c_void_p * 2)()
    t.filter = b"fc1"
    t.events = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    t.capacity = mok.TRACE_MAX + 1
    assert lib.mok_trace_bind(ctypes.byref(t)) == 3
    t.capacity = 1
    assert lib.mok_trace_bind(ctypes.byref(t)) == 0
    assert lib.mok_trace_bind(None) == 0


def test_noalloc_forward_refuses_oversized_workspace_before_launch(mok):
    """mok_moe_forward_noalloc compares the descriptor's forward workspace with its 32 MiB
    device array before touching the device (no GPU needed)."""
    P = ctypes.c_void_p
    d = _d(mok, T=16384, H=7168, E=384, k=8, I=2048)
    assert mok.workspace_query(d)["fwd_ws"] > mok.NOALLOC_WS_BYTES
    w = mok._Weights(4096, 4096, None)
    st = mok._lib.mok_moe_forward_noalloc(ctypes.byref(d.c()), P(4096), P(4096), P(4096), ctypes.byref(w), P(4096),
                                          P(4096), 1 << 40, None)
    assert st == mok.ERR_WORKSPACE


def test_replay_keeps_nothing_for_the_backward(mok):
    """MOK_FLAG_REPLAY: mok_sizes.saved is 0; the forward workspace holds a, u, h instead
    and the backward workspace has room to form them again (bf16, fp32 and MXFP8)."""
    for kw in (dict(), dict(act=mok.F32), dict(gemm=mok.MXFP8, mb_count=4, ring=2)):
        d = _d(mok, T=256, H=256, E=8, k=2, I=128, **kw)
        base = mok.workspace_query(d)
        d.flags |= mok.FLAG_REPLAY
        rp = mok.workspace_query(d)
        es = 4 if d.act == mok.F32 else 2
        act = es * d.R * 3 * d.I
        assert base["saved"] >= act and rp["saved"] == 0
        assert rp["fwd_ws"] >= base["fwd_ws"] + act
        assert rp["bwd_ws"] >= base["bwd_ws"] + act
