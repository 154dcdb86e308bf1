"""Thin Python binding of libmok.so (include/mok.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Tensors are passed as device pointers (``tensor.data_ptr()``) together
with torch's current HIP stream; the library never allocates or synchronises.
If libmok.so is missing this module raises on import -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmok.so")

F32, BF16, MXFP8, MXFP4 = 0, 1, 2, 3
FLAG_WGRAD_F32 = 1
FLAG_WGRAD_DEFER = 2
FLAG_REPLAY = 4
FLAG_FUSED = 8
DTYPES = {"f32": F32, "bf16": BF16, "mxfp8": MXFP8, "mxfp4": MXFP4}
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}

STATUS = {0: "MOK_OK", 1: "MOK_ERR_NULL", 2: "MOK_ERR_ALIGN", 3: "MOK_ERR_SHAPE", 4: "MOK_ERR_DTYPE",
          5: "MOK_ERR_HIP", 6: "MOK_ERR_WORKSPACE", 7: "MOK_ERR_SCHEDULE_MISMATCH"}
ERR_WORKSPACE, ERR_SCHEDULE_MISMATCH = 6, 7
TRACE_MAX = 4096


class MokError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), text))
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("act", ctypes.c_int32), ("gemm", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("tile_m", ctypes.c_int32), ("grid", ctypes.c_int32), ("mb_index", ctypes.c_int32),
                ("mb_count", ctypes.c_int32), ("ring", ctypes.c_int32), ("reserved", ctypes.c_int32)]


MX_FIELDS = ("w1q", "w1s", "w2q", "w2s", "w2tq", "w2ts", "w1tq", "w1ts")


class _MxWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in MX_FIELDS]


class _Weights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("mx", ctypes.POINTER(_MxWeights))]


class _Sizes(ctypes.Structure):
    _fields_ = [("sched", ctypes.c_size_t), ("saved", ctypes.c_size_t), ("fwd_ws", ctypes.c_size_t),
                ("bwd_ws", ctypes.c_size_t)]


class _SchedLayout(ctypes.Structure):
    _fields_ = [("status", ctypes.c_size_t), ("counts", ctypes.c_size_t), ("offsets", ctypes.c_size_t),
                ("tile_start", ctypes.c_size_t), ("num_tiles", ctypes.c_size_t), ("perm", ctypes.c_size_t),
                ("inv", ctypes.c_size_t), ("tiles", ctypes.c_size_t), ("tile_m", ctypes.c_int32),
                ("max_tiles", ctypes.c_int32), ("hash", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


class _Trace(ctypes.Structure):
    _fields_ = [("filter", ctypes.c_char_p), ("events", ctypes.POINTER(ctypes.c_void_p)),
                ("capacity", ctypes.c_int32), ("count", ctypes.c_int32), ("names", ctypes.c_char_p * TRACE_MAX)]


class _SavedLayout(ctypes.Structure):
    _fields_ = [("au_offset", ctypes.c_size_t), ("h_offset", ctypes.c_size_t)]


MX_LAYOUT_FIELDS = ("fwd_slot", "xq", "xs", "hq", "hs", "bwd_slot", "dyq", "dys", "dguq", "dgus", "st_xs", "st_dos",
                    "st_h", "st_dgu", "pofs", "dot", "dots", "ht", "hts", "dgut", "dguts", "xt", "xts")


class _MxLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in MX_LAYOUT_FIELDS] + [("kmax", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmok.so is not built (%s); run `python -m mixture_experts_layer_stable_amd.build`"
                           % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    Z = ctypes.c_size_t
    D = ctypes.POINTER(_Desc)
    sig = {
        "mok_workspace_query": [D, ctypes.POINTER(_Sizes)],
        "mok_schedule_layout_query": [D, ctypes.POINTER(_SchedLayout)],
        "mok_saved_layout_query": [D, ctypes.POINTER(_SavedLayout)],
        "mok_mx_layout_query": [D, ctypes.POINTER(_MxLayout)],
        "mok_route": [D, P, P, P, P, P, P, P],
        "mok_schedule_build": [D, P, P, Z, P],
        "mok_moe_forward": [D, P, P, P, ctypes.POINTER(_Weights), P, P, Z, P, Z, P],
        "mok_moe_forward_noalloc": [D, P, P, P, ctypes.POINTER(_Weights), P, P, Z, P],
        "mok_moe_backward": [D, P, P, P, P, ctypes.POINTER(_Weights), P, P, Z, P, P, P, P, P, P, P, Z, P],
        "mok_trace_bind": [ctypes.POINTER(_Trace)],
        "mok_weights_quantize": [D, P, P, ctypes.POINTER(_MxWeights), P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.mok_status_string.argtypes = [ctypes.c_int]
    lib.mok_status_string.restype = ctypes.c_char_p
    lib.mok_version.argtypes = []
    lib.mok_version.restype = ctypes.c_int32
    return lib


_lib = _load()
EXPORTS = ("mok_workspace_query", "mok_schedule_layout_query", "mok_saved_layout_query", "mok_mx_layout_query",
           "mok_route",
           "mok_schedule_build", "mok_moe_forward", "mok_moe_forward_noalloc", "mok_moe_backward",
           "mok_weights_quantize", "mok_status_string", "mok_version", "mok_trace_bind")
NOALLOC_WS_BYTES = 32 << 20


@dataclass
class Desc:
    T: int
    H: int
    E: int
    k: int
    I: int
    act: int = BF16
    gemm: Optional[int] = None
    flags: int = 0
    tile_m: int = 0
    grid: int = 0
    mb_index: int = 0
    mb_count: int = 1
    ring: int = 1

    def c(self) -> _Desc:
        g = self.act if self.gemm is None else self.gemm
        return _Desc(self.T, self.H, self.E, self.k, self.I, self.act, g, self.flags, self.tile_m, self.grid,
                     self.mb_index, self.mb_count, self.ring, 0)

    @property
    def mx(self) -> bool:
        return self.gemm in (MXFP8, MXFP4)

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def dtype(self) -> torch.dtype:
        return TORCH_DTYPE[self.act]


def _check(st: int, where: str):
    if st != 0:
        raise MokError(st, where, _lib.mok_status_string(st).decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nb(t: Optional[torch.Tensor]) -> int:
    """Bytes of a buffer tensor (0 for None)."""
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def version() -> int:
    return _lib.mok_version()


def workspace_query(d: Desc) -> dict:
    s = _Sizes()
    _check(_lib.mok_workspace_query(ctypes.byref(d.c()), ctypes.byref(s)), "mok_workspace_query")
    return dict(sched=s.sched, saved=s.saved, fwd_ws=s.fwd_ws, bwd_ws=s.bwd_ws)


def schedule_layout_query(d: Desc) -> dict:
    s = _SchedLayout()
    _check(_lib.mok_schedule_layout_query(ctypes.byref(d.c()), ctypes.byref(s)), "mok_schedule_layout_query")
    return {n: getattr(s, n) for n, _ in _SchedLayout._fields_}


def saved_layout_query(d: Desc) -> dict:
    s = _SavedLayout()
    _check(_lib.mok_saved_layout_query(ctypes.byref(d.c()), ctypes.byref(s)), "mok_saved_layout_query")
    return dict(au_offset=s.au_offset, h_offset=s.h_offset)


def mx_layout_query(d: Desc) -> dict:
    s = _MxLayout()
    _check(_lib.mok_mx_layout_query(ctypes.byref(d.c()), ctypes.byref(s)), "mok_mx_layout_query")
    return {n: getattr(s, n) for n, _ in _MxLayout._fields_}


def schedule_views(d: Desc, sched) -> dict:
    """int32 views of the parts of a schedule buffer built for descriptor d (for inspection and tests)."""
    L = schedule_layout_query(d)

    def iv(off, n):
        return sched[off: off + 4 * n].view(torch.int32)

    return dict(counts=iv(L["counts"], d.E), offsets=iv(L["offsets"], d.E + 1),
                tile_start=iv(L["tile_start"], d.E + 1), num_tiles=iv(L["num_tiles"], 1),
                perm=iv(L["perm"], d.R), inv=iv(L["inv"], d.R),
                tiles=iv(L["tiles"], 4 * L["max_tiles"]).view(-1, 4), tile_m=L["tile_m"],
                max_tiles=L["max_tiles"], status=int(iv(L["status"], 1).cpu()[0]))


def route(d: Desc, x, wr, bias, idx, gate, logits=None, stream=None):
    _check(_lib.mok_route(ctypes.byref(d.c()), _p(x), _p(wr), _p(bias), _p(idx), _p(gate), _p(logits),
                          _stream(stream)), "mok_route")


def schedule_build(d: Desc, idx, sched, stream=None):
    _check(_lib.mok_schedule_build(ctypes.byref(d.c()), _p(idx), _p(sched), _nb(sched), _stream(stream)),
           "mok_schedule_build")


def schedule_status(d: Desc, sched) -> int:
    """The schedule header's status word (synchronises on the tensor read): MOK_OK, or
    MOK_ERR_SCHEDULE_MISMATCH once a kernel was handed this table with another descriptor."""
    off = schedule_layout_query(d)["status"]
    return int(sched[off: off + 4].view(torch.int32).cpu()[0])


def check_schedule(d: Desc, sched, where="schedule"):
    """Raise MokError if a forward/backward kernel rejected the schedule (after a sync)."""
    st = schedule_status(d, sched)
    if st != 0:
        raise MokError(st, where, _lib.mok_status_string(st).decode())


class MxWeights:
    """Device tensors of the MX weight orientations (mok_mx_weights), filled by weights_quantize.
    Element bytes [E][rows][K] (MXFP8) or [E][rows][K/2] (MXFP4, two E2M1 codes per byte)."""

    def __init__(self, d: Desc, device="cuda"):
        E, H, I = d.E, d.H, d.I
        u8 = dict(dtype=torch.uint8, device=device)
        q = (lambda k: k // 2) if d.gemm == MXFP4 else (lambda k: k)
        # scales K-tile-major: [E][K/128][rows][4]
        self.w1q, self.w1s = torch.empty(E, 2 * I, q(H), **u8), torch.empty(E, H // 128, 2 * I, 4, **u8)
        self.w2q, self.w2s = torch.empty(E, H, q(I), **u8), torch.empty(E, I // 128, H, 4, **u8)
        self.w2tq, self.w2ts = torch.empty(E, I, q(H), **u8), torch.empty(E, H // 128, I, 4, **u8)
        self.w1tq, self.w1ts = torch.empty(E, H, q(2 * I), **u8), torch.empty(E, 2 * I // 128, H, 4, **u8)

    def c(self) -> _MxWeights:
        return _MxWeights(*[getattr(self, n).data_ptr() for n in MX_FIELDS])


def weights_quantize(d: Desc, w1, w2, mxw: MxWeights, stream=None):
    q = mxw.c()
    _check(_lib.mok_weights_quantize(ctypes.byref(d.c()), _p(w1), _p(w2), ctypes.byref(q), _stream(stream)),
           "mok_weights_quantize")


def _weights(w1, w2, mxw):
    q = None if mxw is None else mxw.c()
    w = _Weights(None if w1 is None else w1.data_ptr(), None if w2 is None else w2.data_ptr(),
                 None if q is None else ctypes.pointer(q))
    return w, q     # q must outlive the call


def moe_forward(d: Desc, sched, x, gate, w1, w2, y, saved, ws, stream=None, mxw: Optional[MxWeights] = None):
    w, _keep = _weights(w1, w2, mxw)
    _check(_lib.mok_moe_forward(ctypes.byref(d.c()), _p(sched), _p(x), _p(gate), ctypes.byref(w), _p(y), _p(saved),
                                _nb(saved), _p(ws), _nb(ws), _stream(stream)), "mok_moe_forward")


def moe_forward_noalloc(d: Desc, sched, x, gate, w1, w2, y, saved, stream=None, mxw: Optional[MxWeights] = None):
    """mok_moe_forward_noalloc: the forward with the library's own device workspace."""
    w, _keep = _weights(w1, w2, mxw)
    _check(_lib.mok_moe_forward_noalloc(ctypes.byref(d.c()), _p(sched), _p(x), _p(gate), ctypes.byref(w), _p(y),
                                        _p(saved), _nb(saved), _stream(stream)), "mok_moe_forward_noalloc")


def moe_backward(d: Desc, sched, x, idx, gate, w1, w2, wr, saved, dy, dx, dw1, dw2, dgate, dwr, ws, stream=None,
                 mxw: Optional[MxWeights] = None):
    w, _keep = _weights(w1, w2, mxw)
    _check(_lib.mok_moe_backward(ctypes.byref(d.c()), _p(sched), _p(x), _p(idx), _p(gate), ctypes.byref(w), _p(wr),
                                 _p(saved), _nb(saved), _p(dy), _p(dx), _p(dw1), _p(dw2), _p(dgate), _p(dwr), _p(ws),
                                 _nb(ws), _stream(stream)), "mok_moe_backward")


class KernelTrace:
    """Bracket launches of one kernel group (or "*") with HIP events (a caller-owned
    mok_trace bound to this thread with mok_trace_bind).

    with KernelTrace("fc1", capacity=64) as tr:
        ... launches ...
    tr.durations_ms()  -> [(name, ms), ...]   (synchronises on the events)
    """

    def __init__(self, name: str, capacity: int = 256):
        self.name = name
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * capacity)]
        for e in self.events:        # materialise the underlying hipEvent_t
            e.record()
        torch.cuda.synchronize()
        self._handles = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
        self._filter = name.encode()
        self._t = _Trace()
        self._t.filter = self._filter
        self._t.events = ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p))
        self._t.capacity = capacity
        self._t.count = 0
        self.capacity = capacity
        self.count = 0
        self.names = []

    def __enter__(self):
        _check(_lib.mok_trace_bind(ctypes.byref(self._t)), "mok_trace_bind")
        return self

    def __exit__(self, *exc):
        _lib.mok_trace_bind(None)
        self.count = self._t.count
        self.names = [self._t.names[i].decode() for i in range(self.count)]
        return False

    def durations_ms(self):
        self.events[2 * max(self.count, 1) - 1].synchronize()
        return [(self.names[i], self.events[2 * i].elapsed_time(self.events[2 * i + 1])) for i in range(self.count)]


# ---------------------------------------------------------------------------
# Convenience: the buffers one layer step needs, and views into them.
# ---------------------------------------------------------------------------

class Buffers:
    """Caller-owned device buffers of one layer step (sizes from mok_workspace_query)."""

    def __init__(self, d: Desc, device="cuda", backward=True, wgrad_f32=False):
        sz = workspace_query(d)
        u8 = dict(dtype=torch.uint8, device=device)
        self.desc = d
        self.sched = torch.empty(max(sz["sched"], 256), **u8)
        self.saved = torch.empty(max(sz["saved"], 256), **u8)
        self.fwd_ws = torch.empty(max(sz["fwd_ws"], 256), **u8)
        self.bwd_ws = torch.empty(max(sz["bwd_ws"], 256), **u8) if backward else None
        f32 = dict(dtype=torch.float32, device=device)
        self.idx = torch.empty(max(d.R, 4), dtype=torch.int32, device=device)[: d.R].view(d.T, d.k)
        self.gate = torch.empty(max(d.R, 4), **f32)[: d.R].view(d.T, d.k)
        self.y = torch.empty(d.T, d.H, dtype=d.dtype, device=device)
        if backward:
            wdt = torch.float32 if (wgrad_f32 or d.act == F32) else d.dtype
            self.dx = torch.empty(d.T, d.H, dtype=d.dtype, device=device)
            self.dgate = torch.empty(max(d.R, 4), **f32)[: d.R].view(d.T, d.k)
            self.dw1 = torch.empty(d.E, 2 * d.I, d.H, dtype=wdt, device=device)
            self.dw2 = torch.empty(d.E, d.H, d.I, dtype=wdt, device=device)
            self.dwr = torch.empty(d.E, d.H, dtype=wdt, device=device)

    def schedule_views(self) -> dict:
        """int32 views of the schedule table's parts (for inspection and tests)."""
        return schedule_views(self.desc, self.sched)

    def saved_views(self) -> dict:
        """a, u [R, I] and h [R, I] in routed-row order (views into `saved`)."""
        L = saved_layout_query(self.desc)
        d = self.desc
        es = 4 if d.act == F32 else 2
        au = self.saved[L["au_offset"]: L["au_offset"] + es * d.R * 2 * d.I].view(d.dtype).view(d.R, 2 * d.I)
        h = self.saved[L["h_offset"]: L["h_offset"] + es * d.R * d.I].view(d.dtype).view(d.R, d.I)
        return dict(a=au[:, : d.I], u=au[:, d.I:], h=h)


def step(d: Desc, buf: Buffers, x, wr, bias, w1, w2, dy=None, stream=None, router_grad=True, mxw=None):
    """route -> schedule -> forward (-> backward): one layer step, all on the GPU."""
    route(d, x, wr, bias, buf.idx, buf.gate, None, stream)
    schedule_build(d, buf.idx, buf.sched, stream)
    moe_forward(d, buf.sched, x, buf.gate, w1, w2, buf.y, buf.saved, buf.fwd_ws, stream, mxw)
    if dy is not None:
        moe_backward(d, buf.sched, x, buf.idx, buf.gate, w1, w2, wr if router_grad else None, buf.saved, dy,
                     buf.dx, buf.dw1, buf.dw2, buf.dgate, buf.dwr if router_grad else None, buf.bwd_ws, stream, mxw)


class StreamedStep:
    """Buffers and call sequence of one streamed MXFP8 step: d.mb_count micro-batches of
    d.T tokens (x, dy are [mb_count*T, H]); route -> schedule -> forward for micro-batches
    0..M-1, then backward for M-1..0, deferring the weight gradients to the last call."""

    def __init__(self, d: Desc, device="cuda", wgrad_f32=False):
        assert d.mx
        self.d = d
        M, T = d.mb_count, d.T
        sz = workspace_query(d)
        u8 = dict(dtype=torch.uint8, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.sched = [torch.empty(max(sz["sched"], 256), **u8) for _ in range(M)]
        self.saved = [torch.empty(max(sz["saved"], 256), **u8) for _ in range(M)]
        self.fwd_ws = torch.empty(max(sz["fwd_ws"], 256), **u8)
        self.bwd_ws = torch.empty(max(sz["bwd_ws"], 256), **u8)
        self.idx = torch.empty(M * T, d.k, dtype=torch.int32, device=device)
        self.gate = torch.empty(M * T, d.k, **f32)
        self.dgate = torch.empty(M * T, d.k, **f32)
        self.y = torch.empty(M * T, d.H, dtype=torch.bfloat16, device=device)
        self.dx = torch.empty(M * T, d.H, dtype=torch.bfloat16, device=device)
        wdt = torch.float32 if wgrad_f32 else torch.bfloat16
        self.dw1 = torch.empty(d.E, 2 * d.I, d.H, dtype=wdt, device=device)
        self.dw2 = torch.empty(d.E, d.H, d.I, dtype=wdt, device=device)
        self.dwr = torch.empty(d.E, d.H, dtype=wdt, device=device)

    def desc(self, m: int, defer: bool = False) -> Desc:
        from dataclasses import replace
        return replace(self.d, mb_index=m, flags=self.d.flags | (FLAG_WGRAD_DEFER if defer else 0))

    def run(self, x, wr, bias, mxw: MxWeights, dy=None, stream=None, router_grad=True):
        d, M, T = self.d, self.d.mb_count, self.d.T
        sl = lambda t, m: t[m * T:(m + 1) * T]
        for m in range(M):
            dm = self.desc(m)
            route(dm, sl(x, m), wr, bias, sl(self.idx, m), sl(self.gate, m), None, stream)
            schedule_build(dm, sl(self.idx, m), self.sched[m], stream)
            moe_forward(dm, self.sched[m], sl(x, m), sl(self.gate, m), None, None, sl(self.y, m), self.saved[m],
                        self.fwd_ws, stream, mxw)
        if dy is None:
            return
        for m in reversed(range(M)):
            dm = self.desc(m, defer=m > 0)
            moe_backward(dm, self.sched[m], sl(x, m), sl(self.idx, m), sl(self.gate, m), None, None,
                         wr if router_grad else None, self.saved[m], sl(dy, m), sl(self.dx, m), self.dw1, self.dw2,
                         sl(self.dgate, m), self.dwr if router_grad else None, self.bwd_ws, stream, mxw)
