"""Shared helpers of the GPU parity tests: run one layer step through the C ABI
and the same step through the oracle, on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
from mixture_experts_layer_stable_amd import inputs

TOL = {"bf16": 5e-3, "f32": 1e-5}
# The same bound for every single row (last-axis vector) of an output, looser than the
# whole-tensor one: a row holds few elements, so one storage-rounding step weighs more
# (largest row errors measured on the small workloads: bf16 6.2e-3, fp32 1.5e-6).
ROW_TOL = {"bf16": 2e-2, "f32": 2e-5}


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        return 0.0 if np.all(got == 0) else float("inf")
    return float(np.linalg.norm(got - ref) / nr)


def rel_fro_rows(got, ref) -> float:
    """Largest relative Frobenius error over the rows (last-axis vectors) of the two
    arrays: a wrong tile, row or column block shows up here even where it moves the
    whole-tensor norm by little. A row whose reference is all zero must be all zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    zero = den == 0
    if np.any(num[zero] > 0):
        return float("inf")
    return float(np.max(num[~zero] / den[~zero])) if np.any(~zero) else 0.0


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Case:
    """Inputs of one workload (full tensors, CPU) plus optional overrides."""

    def __init__(self, w: inputs.Workload, x=None, wr=None, bias="default", w1=None, w2=None, dy=None):
        self.w = w
        self.x = inputs.make_x(w) if x is None else x
        self.wr = inputs.make_wr(w) if wr is None else wr
        self.bias = inputs.make_bias(w) if isinstance(bias, str) else bias
        self.w1 = torch.stack([inputs.make_w1(w, e) for e in range(w.E)]) if w1 is None else w1
        self.w2 = torch.stack([inputs.make_w2(w, e) for e in range(w.E)]) if w2 is None else w2
        self.dy = inputs.make_dy(w) if dy is None else dy


def run_gpu(case: Case, backward=True, tile_m=0, grid=0, router_grad=True, wgrad_f32=False, logits=True,
            replay=False, fused=False):
    from mixture_experts_layer_stable_amd import mok
    w = case.w
    dev = "cuda"
    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.DTYPES[w.act], tile_m=tile_m, grid=grid,
                 flags=(mok.FLAG_WGRAD_F32 if wgrad_f32 else 0) | (mok.FLAG_REPLAY if replay else 0)
                 | (mok.FLAG_FUSED if fused else 0))
    buf = mok.Buffers(d, dev, backward=backward, wgrad_f32=wgrad_f32)
    x = case.x.to(dev)
    wr = case.wr.to(dev)
    bias = None if case.bias is None else case.bias.to(dev)
    w1 = case.w1.to(dev)
    w2 = case.w2.to(dev)
    lg = torch.empty(w.T, w.E, dtype=torch.float32, device=dev) if logits else None
    mok.route(d, x, wr, bias, buf.idx, buf.gate, lg)
    mok.schedule_build(d, buf.idx, buf.sched)
    mok.moe_forward(d, buf.sched, x, buf.gate, w1, w2, buf.y, buf.saved, buf.fwd_ws)
    out = {}
    if backward:
        dy = case.dy.to(dev)
        mok.moe_backward(d, buf.sched, x, buf.idx, buf.gate, w1, w2, wr if router_grad else None, buf.saved, dy,
                         buf.dx, buf.dw1, buf.dw2, buf.dgate, buf.dwr if router_grad else None, buf.bwd_ws)
    torch.cuda.synchronize()
    mok.check_schedule(d, buf.sched, "layer step")
    sv = buf.schedule_views()
    out.update(idx=buf.idx.cpu().numpy(), gate=buf.gate.cpu().numpy(), y=buf.y.cpu(),
               counts=sv["counts"].cpu().numpy(), offsets=sv["offsets"].cpu().numpy(),
               tile_start=sv["tile_start"].cpu().numpy(), num_tiles=int(sv["num_tiles"].cpu()[0]),
               perm=sv["perm"].cpu().numpy(), inv=sv["inv"].cpu().numpy(),
               tiles=sv["tiles"].cpu().numpy(), tile_m=sv["tile_m"])
    if logits:
        out["logits"] = lg.cpu().numpy()
    if not replay:
        saved = buf.saved_views()
        out.update(a=saved["a"].cpu(), u=saved["u"].cpu(), h=saved["h"].cpu())
    if backward:
        out.update(dx=buf.dx.cpu(), dw1=buf.dw1.cpu(), dw2=buf.dw2.cpu(), dgate=buf.dgate.cpu().numpy())
        if router_grad:
            out["dwr"] = buf.dwr.cpu()
    return out


def run_oracle(case: Case, backward=True, BM=32, router_grad=True, wfmt=None):
    w = case.w
    x = case.x.float().numpy()
    wr = case.wr.float().numpy()
    bias = None if case.bias is None else case.bias.numpy()
    z, idx, g = orc.route(x, wr, w.k, bias)
    sc = orc.schedule(idx, w.E, BM)
    W = orc.DenseWeights(case.w1.float().numpy(), case.w2.float().numpy())
    fmt = w.act
    fwd = orc.forward(x, W, idx, g, fmt, w.E, w.I)
    out = dict(z=z, idx=idx, gate=g, sched=sc, fwd=fwd)
    if backward:
        out["bwd"] = orc.backward(x, W, wr, idx, g, fwd, case.dy.float().numpy(), fmt, w.I,
                                  wfmt=wfmt or fmt, router=router_grad)
    return out


def oracle_step_parallel(x, W, wr, idx, gate, dy, E, I, fmt="bf16", mx=False, workers=8):
    """The oracle's forward and backward over all experts that have slots, evaluated as expert
    chunks in threads (numpy releases the GIL in its large array operations) and merged;
    then the token side: the slot-order combine and the router backward / dX reduction
    (oracle.combine, oracle.reduce_backward). Bit for bit the oracle's whole-step result,
    which a CPU test checks; the full-size GPU tests use it to keep the oracle's passes over
    hundreds of experts within minutes. mx: False, or the MX element format ('e4m3', 'e2m1';
    True means 'e4m3')."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=max(1, 16 // workers)):
        return _oracle_step_parallel(x, W, wr, idx, gate, dy, E, I, fmt, mx, workers, ThreadPoolExecutor)


def _oracle_step_parallel(x, W, wr, idx, gate, dy, E, I, fmt, mx, workers, ThreadPoolExecutor):
    present = sorted(set(np.asarray(idx).ravel().tolist()))
    chunks = [c for c in (present[i::workers] for i in range(workers)) if c]
    flat = np.asarray(idx).ravel()

    def rows_of(ch):
        return np.nonzero(np.isin(flat, ch))[0]

    mxf = "e4m3" if mx is True else mx

    def fwd(ch):
        if mx:
            return ch, orc.mx.forward_mx(x, W, idx, gate, E, I, experts=ch, fmt=mxf)
        return ch, orc.forward(x, W, idx, gate, fmt, E, I, experts=ch)

    with ThreadPoolExecutor(len(chunks)) as ex:
        fparts = list(ex.map(fwd, chunks))
    f = {key: np.full_like(fparts[0][1][key], np.nan) for key in fparts[0][1]}
    for ch, part in fparts:
        r = rows_of(ch)
        for key in f:
            f[key][r] = part[key][r]
    f["y"] = orc.combine(f["p"], gate, "bf16" if mx else fmt)

    def bwd(ch):
        if mx:
            return ch, orc.mx.backward_mx(x, W, wr, idx, gate, f, dy, I, experts=ch, fmt=mxf)
        return ch, orc.backward(x, W, wr, idx, gate, f, dy, fmt, I, experts=ch)

    with ThreadPoolExecutor(len(chunks)) as ex:
        bparts = list(ex.map(bwd, chunks))
    T, k = np.asarray(idx).shape
    b = dict(dgate=np.full(T * k, np.nan), dgu=np.full((T * k, 2 * I), np.nan),
             q=np.full((T * k, np.asarray(x).shape[1]), np.nan), dw1={}, dw2={})
    for ch, part in bparts:
        r = rows_of(ch)
        b["dgate"][r] = part["dgate"].ravel()[r]
        b["dgu"][r] = part["dgu"][r]
        b["q"][r] = part["q"][r]
        b["dw1"].update(part["dw1"])
        b["dw2"].update(part["dw2"])
    b["dgate"] = b["dgate"].reshape(T, k)
    act = "bf16" if mx else fmt
    b.update(orc.reduce_backward(x, wr, idx, gate, b["dgate"], b["q"], act, act))
    return f, b
