"""Oracle MX quantisation (MXFP8, MXFP4) and the MX layer step. TEST INFRASTRUCTURE ONLY.

The expert GEMMs run on MXFP8 operands (dothoosh.com MoK page, "Technical details of the
MoK mechanism": the megakernel supports BF16 and MXFP8). Format, from the OCP Microscaling
(MX) specification v1.0: blocks of 32 consecutive elements along the GEMM's K share one
E8M0 scale 2^s; elements are FP8 E4M3 (max normal 448, subnormals down to 2^-9).

Quantisation of one block (values v, all exactly representable in bf16/fp32):
  amax = max |v|;  if amax == 0: s = -127 and every element is 0;
  else s = floor(log2 amax) - 8 (8 = exponent of E4M3's largest normal), clamped to
  [-127, 127]; element = E4M3 round-to-nearest-even of v / 2^s, saturated to +-448.
Dequantisation is exact: element * 2^s.

MXFP4 (the narrower expert GEMMs the pages name as Cursor's earlier work, aikraft.ru MoK
article, section 03, with no detail): the same spec's FP4 E2M1 elements (1 mantissa bit,
largest normal 6 = 1.5 * 2^2, smallest normal 1, subnormal 0.5) under the same E8M0
block scale, s = floor(log2 amax) - 2 (2 = exponent of E2M1's largest normal), elements
rounded to nearest even and saturated to +-6 (the format has no infinities); the
quantisation points are MXFP8's. `fmt` selects the element format ('e4m3' or 'e2m1').

Quantisation points of the step (each GEMM operand along that GEMM's K):
  fc1  x rows along H,  W1 rows along H
  fc2  h rows (bf16 as stored) along I,  W2 rows along I
  dh   dY rows along H,  W2^T rows (columns of W2) along H
  dx   dGU rows (bf16 as stored) along 2I,  W1^T rows along 2I
  dw2  dO = bf16(g*dY) and h along tokens
  dw1  dGU and x along tokens
For the weight gradients, token blocks start at each expert's first row of the whole
step (all micro-batches, in token order) and the last block is padded with zeros; the
`segments` argument of backward_mx restarts blocks at other segment boundaries instead. The gate gradient is
g' = <dA, h> with dA the dh GEMM result (the fused SonicMoE-style form; with quantised
operands it is the method's definition).
"""
from __future__ import annotations

import numpy as np

from .moe import bf16_round, combine, reduce_backward, round_to, sigmoid, silu, _slots_by_expert

E4M3_MAX = 448.0
E2M1_MAX = 6.0
MX_BLOCK = 32

# element format: (exponent of the largest normal, exponent of the smallest normal,
# mantissa bits, largest magnitude)
FORMATS = {"e4m3": (8, -6, 3, E4M3_MAX), "e2m1": (2, 0, 1, E2M1_MAX)}


def elem_round(v, fmt="e4m3"):
    """Round-to-nearest-even onto the element format (normals with `mbits` mantissa bits
    from 2^emin up, subnormals spaced like the smallest binade), saturating at +-max."""
    _, emin, mbits, vmax = FORMATS[fmt]
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                                   # a = m * 2^e, 0.5 <= m < 1
    q = np.exp2(np.maximum(e - 1, emin).astype(np.float64) - mbits)
    r = np.rint(v / q) * q
    return np.clip(np.where(a == 0, 0.0 * v, r), -vmax, vmax)


def e4m3_round(v):
    """FP8 E4M3: 3 mantissa bits, min normal 2^-6, subnormal step 2^-9, max 448."""
    return elem_round(v, "e4m3")


def e2m1_round(v):
    """FP4 E2M1: 1 mantissa bit, min normal 1, subnormal step 0.5, max 6."""
    return elem_round(v, "e2m1")


def mx_quantize(v, axis=-1, fmt="e4m3"):
    """Blocks of 32 along `axis` (its length must be a multiple of 32).
    Returns (elements as float64 values of the element format, scale exponents s as int,
    same shape with the axis divided by 32)."""
    emax = FORMATS[fmt][0]
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    K = v.shape[-1]
    assert K % MX_BLOCK == 0, K
    blk = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, e = np.frexp(amax)
    s = np.clip(e - 1 - emax, -127, 127)
    s = np.where(amax == 0, -127, s).astype(np.int64)
    el = elem_round(blk / np.exp2(s.astype(np.float64))[..., None], fmt)
    el = np.where((amax == 0)[..., None], 0.0, el)
    return np.moveaxis(el.reshape(v.shape), -1, axis), np.moveaxis(s, -1, axis)


def mx_dequantize(el, s, axis=-1):
    el = np.moveaxis(np.asarray(el, np.float64), axis, -1)
    s = np.moveaxis(np.asarray(s), axis, -1)
    K = el.shape[-1]
    out = el.reshape(el.shape[:-1] + (K // MX_BLOCK, MX_BLOCK)) * np.exp2(s.astype(np.float64))[..., None]
    return np.moveaxis(out.reshape(el.shape), -1, axis)


def mx(v, axis=-1, fmt="e4m3"):
    """Quantise then dequantise (the value an MX GEMM operand stands for)."""
    return mx_dequantize(*mx_quantize(v, axis, fmt), axis=axis)


def mx_token_blocks(rows, seg_lengths, fmt="e4m3"):
    """Quantise token-major rows [n, F] along tokens, blocks of 32 starting at each
    segment's first row, zero-padded at each segment's end; returns the dequantised
    rows (same shape)."""
    out = np.empty_like(np.asarray(rows, np.float64))
    pos = 0
    for n in seg_lengths:
        if n == 0:
            continue
        pad = -(-n // MX_BLOCK) * MX_BLOCK
        blk = np.zeros((pad, rows.shape[1]))
        blk[:n] = rows[pos:pos + n]
        out[pos:pos + n] = mx(blk, axis=0, fmt=fmt)[:n]
        pos += n
    return out


def forward_mx(x, weights, idx, gate, E: int, I: int, experts=None, fmt="e4m3") -> dict:
    """MX expert GEMMs (element format `fmt`), bf16 storage: same outputs as
    moe.forward(fmt='bf16') with every GEMM operand quantised along its K. ``experts``
    restricts the work to a subset of experts (other slots stay NaN and y is not formed)."""
    q = lambda v, axis=-1: mx(v, axis, fmt)
    x = np.asarray(x, np.float64)
    T, H = x.shape
    k = idx.shape[1]
    R = T * k
    a_s = np.full((R, I), np.nan)
    u_s = np.full((R, I), np.nan)
    h_s = np.full((R, I), np.nan)
    p = np.full((R, H), np.nan)
    by_e = _slots_by_expert(idx, E)
    for e in (range(E) if experts is None else experts):
        s = by_e[e]
        if s.size == 0:
            continue
        X = q(x[s // k])
        W1 = q(weights.w1(e))
        A = X @ W1[:I].T
        U = X @ W1[I:].T
        Hh = bf16_round(silu(A) * U)
        O = q(Hh) @ q(weights.w2(e)).T
        a_s[s], u_s[s], h_s[s], p[s] = bf16_round(A), bf16_round(U), Hh, bf16_round(O)
    if experts is not None:
        return dict(a=a_s, u=u_s, h=h_s, p=p)
    return dict(a=a_s, u=u_s, h=h_s, p=p, y=combine(p, gate, "bf16"))


def backward_mx(x, weights, wr, idx, gate, fwd, dy, I: int, segments=None, router=True, experts=None,
                wfmt: str = "bf16", fmt: str = "e4m3") -> dict:
    """Gradients with MX expert GEMMs (element format `fmt`). `segments[e]` lists the lengths of expert e's
    row segments in slot order, token blocks restarting at each (default: one segment,
    the expert's rows of the whole step). ``experts`` restricts the work to a subset of
    experts: only their d-gates, dGU, partial rows and weight gradients are formed.
    ``wfmt`` is the storage format of dW1, dW2, dWr ('bf16', or 'f32' for weight
    gradients kept in fp32); every other stored value is bf16."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    g = np.asarray(gate, np.float64)
    T, H = x.shape
    k = idx.shape[1]
    E = np.asarray(wr).shape[0]
    R = T * k
    gf = g.ravel()
    q = lambda v, axis=-1: mx(v, axis, fmt)
    gp = np.full(R, np.nan)
    dgu = np.full((R, 2 * I), np.nan)
    qp = np.full((R, H), np.nan)
    dw1, dw2 = {}, {}
    by_e = _slots_by_expert(idx, E)
    for e in (range(E) if experts is None else experts):
        s = by_e[e]
        if s.size == 0:
            dw1[e], dw2[e] = np.zeros((2 * I, H)), np.zeros((H, I))
            continue
        t = s // k
        W1 = weights.w1(e)
        W2 = weights.w2(e)
        dA = q(dy[t]) @ q(W2, axis=0)                    # W2^T rows (columns of W2) along H
        hh = fwd["h"][s]
        gp[s] = np.einsum("ri,ri->r", dA, hh)
        dh = gf[s][:, None] * dA
        a, u = fwd["a"][s], fwd["u"][s]
        sg = sigmoid(a)
        G = bf16_round(np.concatenate([dh * u * sg * (1.0 + a * (1.0 - sg)), dh * (a * sg)], axis=1))
        dgu[s] = G
        qp[s] = bf16_round(q(G) @ q(W1, axis=0))         # W1^T rows along 2I
        seg = [s.size] if segments is None else segments[e]
        dO = bf16_round(gf[s][:, None] * dy[t])
        dw2[e] = round_to(mx_token_blocks(dO, seg, fmt).T @ mx_token_blocks(hh, seg, fmt), wfmt)
        dw1[e] = round_to(mx_token_blocks(G, seg, fmt).T @ mx_token_blocks(x[t], seg, fmt), wfmt)
    if experts is not None:
        return dict(dgate=gp.reshape(T, k), dgu=dgu, dw1=dw1, dw2=dw2, q=qp)
    out = dict(dgate=gp.reshape(T, k), dgu=dgu, dw1=dw1, dw2=dw2, q=qp)
    out.update(reduce_backward(x, wr, idx, gate, gp.reshape(T, k), qp, "bf16", wfmt, router))
    return out
