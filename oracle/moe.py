"""Oracle: plain CPU (numpy, fp64) MoE layer step. TEST INFRASTRUCTURE ONLY.

Conventions
-----------
* Token t has k routed slots; flat slot s = t*k + j, j = 0..k-1 in slot order.
* x [T,H], wr [E,H], W1[e] [2I,H] (rows 0..I-1 gate, I..2I-1 up), W2[e] [H,I].
* Every floating result is accumulated in fp64. ``fmt`` names the storage
  format of activations ('f32', 'bf16' or 'exact'): values the layer keeps
  in memory (saved a/u/h, per-slot partials, dGU, outputs) are rounded to it
  once, with round-to-nearest-even, at the point the layer stores them.
  'exact' keeps everything in fp64 (used by the autograd/finite-difference
  pins).
* ``weights`` is any object with methods w1(e) -> [2I,H] and w2(e) -> [H,I]
  returning float64 arrays, so experts can be produced on demand.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

__all__ = [
    "build_oracle", "round_to", "bf16_round", "router_logits", "router_logits_exact", "select_topk",
    "topk_gates", "route", "schedule", "forward", "backward", "DenseWeights", "silu", "sigmoid", "combine",
    "reduce_backward",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libmok_oracle.so")


def build_oracle(force: bool = False) -> str:
    """Compile the oracle's C part (router logits) with gcc; no fast-math, no contraction."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-o", tmp, os.path.join(_HERE, "router.c"), "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _clib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build_oracle())
        _lib.oracle_router_logits.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib.oracle_router_logits.restype = None
    return _lib


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------

def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to even.

    bfloat16 has fp32's exponent range and an 8-bit significand, so the
    spacing at |v| in [2^e', 2^(e'+1)) is 2^(e'-7), never finer than the
    smallest subnormal 2^-133.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    q = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    r = np.rint(v / q) * q                   # np.rint rounds half to even
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    return np.where(np.isfinite(v), r, v)


def round_to(v: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "exact":
        return np.asarray(v, dtype=np.float64)
    if fmt == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_round(v)
    raise ValueError(fmt)


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    return a * sigmoid(a)


class DenseWeights:
    """Expert weights held as dense arrays W1 [E,2I,H], W2 [E,H,I] (converted to fp64)."""

    def __init__(self, w1, w2):
        self._w1 = np.asarray(w1)
        self._w2 = np.asarray(w2)

    def w1(self, e):
        return self._w1[e].astype(np.float64)

    def w2(self, e):
        return self._w2[e].astype(np.float64)


# ----------------------------------------------------------------------------
# Routing: kwkr.cn explainer section 4.1 (top-k gating); tie rule and gate
# normalisation as stated for this layer: ties go to the lower expert index,
# gates are a softmax over the k selected logits (equal to the full softmax
# renormalised over the top k).
# ----------------------------------------------------------------------------

def router_logits(x, wr, bias=None) -> np.ndarray:
    """fp32 logits z [T,E] with the fixed fma order of router.c (routing decisions are integers)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    wr = np.ascontiguousarray(np.asarray(wr, dtype=np.float32))
    T, H = x.shape
    E = wr.shape[0]
    z = np.empty((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
    _clib().oracle_router_logits(T, H, E, x.ctypes.data, wr.ctypes.data,
                                 None if b is None else b.ctypes.data, z.ctypes.data)
    return z


def router_logits_exact(x, wr, bias=None) -> np.ndarray:
    """fp64 logits x . wr^T (+ bias), for the derivative pins."""
    z = np.asarray(x, np.float64) @ np.asarray(wr, np.float64).T
    if bias is not None:
        z = z + np.asarray(bias, np.float64)[None, :]
    return z


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """idx [T,k] int32: the k largest logits per token, slot 0 largest.

    Total order: larger value first; equal values (so -0 == +0) -> lower
    expert index first; NaN ranks below every number.
    """
    z = np.asarray(z)
    T, E = z.shape
    nan = np.isnan(z)
    key = np.where(nan, 0.0, -z.astype(np.float64))     # ascending key = descending value
    eidx = np.broadcast_to(np.arange(E), (T, E))
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((eidx[t], key[t], nan[t]))   # last key is primary
        idx[t] = order[:k]
    return idx


def topk_gates(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g [T,k] fp64: softmax over the selected logits, in slot order."""
    zs = np.take_along_axis(np.asarray(z, np.float64), idx.astype(np.int64), axis=1)
    ex = np.exp(zs - zs[:, :1])
    den = np.zeros(zs.shape[0])
    for j in range(zs.shape[1]):
        den = den + ex[:, j]
    return ex / den[:, None]


def route(x, wr, k, bias=None, exact=False):
    """(z, idx, gate) for every token."""
    z = router_logits_exact(x, wr, bias) if exact else router_logits(x, wr, bias)
    idx = select_topk(z, k)
    return z, idx, topk_gates(z, idx)


# ----------------------------------------------------------------------------
# Schedule: dothoosh.com page, "Technical details of the MoK mechanism": one
# schedule table drives dispatch, combine, reverse-combine and reverse-
# dispatch. It is a stable sort of the T*k slots by expert.
# ----------------------------------------------------------------------------

def schedule(idx: np.ndarray, E: int, BM: int) -> dict:
    """counts [E], offsets [E+1], perm [R] (routed row -> slot), inv [R] (slot -> row),
    tiles [n,3] = (expert, first row, rows) with rows <= BM, experts ascending."""
    flat = np.asarray(idx, dtype=np.int64).ravel()
    R = flat.size
    counts = np.zeros(E, dtype=np.int64)
    perm = np.empty(R, dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    pos = 0
    tiles = []
    for e in range(E):
        slots = np.nonzero(flat == e)[0]            # ascending slot order = stable
        c = slots.size
        counts[e] = c
        offsets[e] = pos
        perm[pos:pos + c] = slots
        for m in range(0, c, BM):
            tiles.append((e, pos + m, min(BM, c - m)))
        pos += c
    offsets[E] = pos
    assert pos == R, "slots routed to experts outside [0, E)"
    inv = np.empty(R, dtype=np.int64)
    inv[perm] = np.arange(R)
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv,
                tiles=np.asarray(tiles, dtype=np.int64).reshape(-1, 3))


# ----------------------------------------------------------------------------
# Forward: SwiGLU expert FFN (dothoosh.com page, "Technical details": SwiGLU
# backward implies a SwiGLU expert), weighted combine in slot order.
# ----------------------------------------------------------------------------

def _slots_by_expert(idx, E):
    flat = np.asarray(idx, dtype=np.int64).ravel()
    return [np.nonzero(flat == e)[0] for e in range(E)]


def forward(x, weights, idx, gate, fmt: str, E: int, I: int, experts=None) -> dict:
    """Per-slot a, u, h (stored), o (fp64), p (stored partial) and y [T,H] (stored).

    For slot s = t*k+j routed to e:  a = W1[e,:I] x_t,  u = W1[e,I:] x_t,
    h = silu(a) * u,  o = W2[e] h.  y_t = sum_j g_tj * p_tj (slot order).
    ``experts`` restricts the work to a subset of experts (slots of other
    experts are left NaN and y is then not formed).
    """
    x = np.asarray(x, np.float64)
    T, H = x.shape
    k = idx.shape[1]
    R = T * k
    a_s = np.full((R, I), np.nan)
    u_s = np.full((R, I), np.nan)
    h_s = np.full((R, I), np.nan)
    o = np.full((R, H), np.nan)
    p = np.full((R, H), np.nan)
    by_e = _slots_by_expert(idx, E)
    todo = range(E) if experts is None else experts
    for e in todo:
        s = by_e[e]
        if s.size == 0:
            continue
        X = x[s // k]
        W1 = weights.w1(e)
        A = X @ W1[:I].T
        U = X @ W1[I:].T
        Hh = round_to(silu(A) * U, fmt)
        O = Hh @ weights.w2(e).T
        a_s[s] = round_to(A, fmt)
        u_s[s] = round_to(U, fmt)
        h_s[s] = Hh
        o[s] = O
        p[s] = round_to(O, fmt)
    out = dict(a=a_s, u=u_s, h=h_s, o=o, p=p)
    if experts is None:
        out["y"] = combine(p, gate, fmt)
    return out


def combine(p, gate, fmt: str) -> np.ndarray:
    """Push combine: y_t = sum_{j=0..k-1} g_tj * p_{t*k+j} in slot order, stored in fmt.
    p [T*k, H] holds every slot's stored partial row."""
    g = np.asarray(gate, np.float64)
    T, k = g.shape
    y = np.zeros((T, np.asarray(p).shape[1]))
    for j in range(k):
        y = y + g[:, j:j + 1] * p[j::k]
    return round_to(y, fmt)


# ----------------------------------------------------------------------------
# Backward: reverse-combine (gather dY to the routed rows), SwiGLU backward
# with the router-weight (gate) gradient fused in SonicMoE-style
# (dothoosh.com page, "Technical details"), reverse-dispatch (dX partials back
# to the token, reduced in slot order), weight gradients, router backward.
# ----------------------------------------------------------------------------

def backward(x, weights, wr, idx, gate, fwd, dy, fmt: str, I: int, wfmt: str = None,
             router: bool = True, experts=None) -> dict:
    """Gradients of L = <dY, y>.

    per slot s = t*k+j routed to e, with stored a, u, h from the forward:
      g'_s  = <dY_t, o_s>                      (d-gate; o = W2[e] h unrounded)
      dA    = W2[e]^T dY_t ;  dh = g_s dA
      da    = dh * u * sig(a) * (1 + a (1 - sig(a))) ;  du = dh * silu(a)
      dGU_s = [da, du]  (stored)
      q_s   = W1[e]^T dGU_s  (stored partial)
      dO_s  = g_s dY_t (stored, the operand of dW2)
    dW1[e] = sum_s dGU_s x_t^T ; dW2[e] = sum_s dO_s h_s^T   (rounded to wfmt)
    dz_s = g_s (g'_s - sum_i g_ti g'_ti)   (softmax over the selected logits)
    dWr[e] = sum_{s: idx=e} dz_s x_t ;  dX_t = sum_j q_tj + sum_j dz_tj Wr[idx_tj]
    """
    wfmt = fmt if wfmt is None else wfmt
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    g = np.asarray(gate, np.float64)
    T, H = x.shape
    k = idx.shape[1]
    E = np.asarray(wr).shape[0]
    R = T * k
    gf = g.ravel()
    gp = np.full(R, np.nan)
    dgu = np.full((R, 2 * I), np.nan)
    q = np.full((R, H), np.nan)
    dw1 = {}
    dw2 = {}
    by_e = _slots_by_expert(idx, E)
    todo = range(E) if experts is None else experts
    for e in todo:
        s = by_e[e]
        if s.size == 0:
            dw1[e] = np.zeros((2 * I, H))
            dw2[e] = np.zeros((H, I))
            continue
        t = s // k
        W1 = weights.w1(e)
        W2 = weights.w2(e)
        dY = dy[t]
        gp[s] = np.einsum("rh,rh->r", dY, fwd["o"][s])
        dA = dY @ W2
        dh = gf[s][:, None] * dA
        a = fwd["a"][s]
        u = fwd["u"][s]
        sg = sigmoid(a)
        da = dh * u * sg * (1.0 + a * (1.0 - sg))
        du = dh * (a * sg)
        G = round_to(np.concatenate([da, du], axis=1), fmt)
        dgu[s] = G
        q[s] = round_to(G @ W1, fmt)
        dO = round_to(gf[s][:, None] * dY, fmt)
        dw1[e] = round_to(G.T @ x[t], wfmt)
        dw2[e] = round_to(dO.T @ fwd["h"][s], wfmt)
    out = dict(dgate=gp.reshape(T, k), dgu=dgu, q=q, dw1=dw1, dw2=dw2)
    if experts is not None:
        return out
    out.update(reduce_backward(x, wr, idx, gate, gp.reshape(T, k), q, fmt, wfmt, router))
    return out


def reduce_backward(x, wr, idx, gate, dgate, q, fmt: str, wfmt: str, router: bool = True) -> dict:
    """The token side of the backward once every slot's d-gate g' and stored partial row
    q are known: dz_s = g_s (g'_s - sum_i g_ti g'_ti) (softmax over the selected logits),
    dX_t = sum_j q_tj (+ sum_j dz_tj Wr[idx_tj]) in slot order, stored in fmt, and
    dWr[e] = sum over e's slots of dz_s x_t, stored in wfmt (only with router)."""
    x = np.asarray(x, np.float64)
    g = np.asarray(gate, np.float64)
    gpk = np.asarray(dgate, np.float64)
    T, H = x.shape
    k = idx.shape[1]
    E = np.asarray(wr).shape[0]
    ssum = np.zeros(T)
    for j in range(k):
        ssum = ssum + g[:, j] * gpk[:, j]
    dz = g * (gpk - ssum[:, None])
    out = dict(dz=dz)
    acc = np.zeros((T, H))
    for j in range(k):
        acc = acc + q[j::k]
    if router:
        wr64 = np.asarray(wr, np.float64)
        for j in range(k):
            acc = acc + dz[:, j:j + 1] * wr64[idx[:, j]]
        dwr = np.zeros((E, H))
        dzf = dz.ravel()
        for e, s in enumerate(_slots_by_expert(idx, E)):
            if s.size:
                dwr[e] = dzf[s] @ x[s // k]
        out["dwr"] = round_to(dwr, wfmt)
    out["dx"] = round_to(acc, fmt)
    return out
