"""GPU parity of the MXFP4 path (FP4 E2M1 elements, two per byte, under the E8M0 scale
of 32-element blocks along each GEMM's K), against the oracle's MX step with
fmt='e2m1':

* the weight quantisers (four orientations), bit for bit, on weights with planted edge
  blocks (zero block, tiny block, saturation, subnormal ties);
* the layer step (route, schedule, forward, backward): rel. Frobenius <= TOL_MX4;
* the step's quantisers (x, dY rows; the fc1 / dh epilogue quantisers of h and dGU; the
  flush's token-axis operands in 256-row segments) bit for bit on the blocks whose bf16
  inputs the GPU and the oracle share;
* streamed == whole batch, bit for bit; an empty batch writes zero weight gradients.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from harness import np64, rel_fro, rel_fro_rows
from mixture_experts_layer_stable_amd import inputs
from test_gpu_mx import _bf16_rows, _case, _compare_blocks, _kmaj, _oracle, _run_streamed, _run_whole

pytestmark = pytest.mark.gpu

DEV = "cuda"
# A bf16 value that the GPU's fp32 GEMM rounds differently from the fp64 oracle moves an
# E2M1 element by a whole step (up to a quarter of its magnitude) when it sits at a
# rounding boundary, against an eighth of that for E4M3; the bound is the MXFP8 one
# doubled.
TOL_MX4 = 4e-2
ROW_TOL_MX = 0.15  # every single row, as for MXFP8 (largest measured 2.4e-2)
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def _mok():
    from mixture_experts_layer_stable_amd import mok
    return mok


def _decode_e2m1(t: torch.Tensor) -> np.ndarray:
    b = t.cpu().numpy().astype(np.uint8).ravel()
    codes = np.stack([b & 15, b >> 4], axis=-1).ravel()   # even element in the low nibble
    return E2M1[codes]


def _edge_weights(E, rows, cols, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((E, rows, cols)) * np.exp2(rng.integers(-40, 41, (E, rows // 32, 1, cols // 32, 1))
                                                      ).repeat(32, 2).repeat(32, 4).reshape(E, rows, cols)
    w[0, :32, :32] = 0.0                                  # all-zero block (both orientations)
    w[0, 32:64, :] *= 2.0**-120                           # tiny: scale clamps at 2^-127
    w[-1, -32:, -32:] = 1.9 * 2.0**10                     # elements 7.6 under the block max 2^10: saturate to 6
    w[-1, -1, -1] = 2.0**10                               # block max sets the scale
    w[1, 5, :] = 0.25 * (1 + 2 * (np.arange(cols) % 2))   # E2M1 ties (0.25, 0.75) under ...
    w[1, 5, ::32] = 4.0                                   # ... a block max of 4 (scale 1)
    return torch.from_numpy(w).to(torch.bfloat16)


def test_weights_quantize_bit_exact_mx4():
    mok = _mok()
    E, H, I = 3, 256, 256
    d = mok.Desc(64, H, E, 2, I, act=mok.BF16, gemm=mok.MXFP4)
    w1 = _edge_weights(E, 2 * I, H, 1)
    w2 = _edge_weights(E, H, I, 2)
    q = mok.MxWeights(d, DEV)
    mok.weights_quantize(d, w1.to(DEV), w2.to(DEV), q)
    torch.cuda.synchronize()
    W1 = w1.double().numpy()
    W2 = w2.double().numpy()
    cases = {
        "w1": (q.w1q, q.w1s, W1),                                  # [E][2I][H] along H
        "w2": (q.w2q, q.w2s, W2),                                  # [E][H][I] along I
        "w2t": (q.w2tq, q.w2ts, np.swapaxes(W2, 1, 2)),            # [E][I][H] along H
        "w1t": (q.w1tq, q.w1ts, np.swapaxes(W1, 1, 2)),            # [E][H][2I] along 2I
    }
    for name, (tq, ts, ref) in cases.items():
        el, s = orc.mx.mx_quantize(ref, -1, "e2m1")
        kt = ts.cpu().numpy().astype(np.int64)
        got_s = np.ascontiguousarray(kt.transpose(0, 2, 1, 3)).reshape(s.shape) - 127
        np.testing.assert_array_equal(got_s, s, err_msg=name + " scales")
        np.testing.assert_array_equal(_decode_e2m1(tq).reshape(el.shape), el, err_msg=name + " elements")


MX4_CASES = {
    "small": inputs.replace(inputs.WORKLOADS["small_bf16"], gemm="mxfp4"),
    "imbalanced": inputs.replace(inputs.WORKLOADS["imbalanced_bf16"], gemm="mxfp4"),
}


def _parity(w, tile_m=0, full=True):
    mok = _mok()
    x, dy, wr, b, w1, w2 = _case(w)
    g = _run_whole(w, x, dy, wr, b, w1, w2, tile_m=tile_m, gemm=mok.MXFP4)
    idx, gate, f, bw = _oracle(w, x, dy, wr, b, w1, w2, fmt="e2m1")
    np.testing.assert_array_equal(g["idx"], idx)
    errs = {
        "y": rel_fro(np64(g["y"]), f["y"]),
        "dx": rel_fro(np64(g["dx"]), bw["dx"]),
        "dgate": rel_fro(g["dgate"].numpy(), bw["dgate"]),
        "dw1": rel_fro(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
        "dw2": rel_fro(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
        "dwr": rel_fro(np64(g["dwr"]), bw["dwr"]),
    }
    if full:
        perm = g["perm"].numpy()
        errs.update(a=rel_fro(np64(g["a"]), f["a"][perm]), u=rel_fro(np64(g["u"]), f["u"][perm]),
                    h=rel_fro(np64(g["h"]), f["h"][perm]))
    print("rel. Frobenius:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL_MX4, (k, v)
    rows = {
        "y": rel_fro_rows(np64(g["y"]), f["y"]),
        "dx": rel_fro_rows(np64(g["dx"]), bw["dx"]),
        "dw1": rel_fro_rows(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
        "dw2": rel_fro_rows(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
        "dwr": rel_fro_rows(np64(g["dwr"]), bw["dwr"]),
    }
    print("largest row error:", {k: "%.2e" % v for k, v in rows.items()}, flush=True)
    for k, v in rows.items():
        assert v <= ROW_TOL_MX, ("row", k, v)


@pytest.mark.parametrize("name,tile_m", [("small", 0), ("imbalanced", 0), ("imbalanced", 64)])
def test_mx4_step_parity(name, tile_m):
    print("case MXFP4", name, "tile_m", tile_m, flush=True)
    _parity(MX4_CASES[name], tile_m)


def test_mx4_ragged_odd_shape():
    """T = 300, k = 3 of E = 5 experts: segments of no tile multiple, token-block tails."""
    w = inputs.replace(MX4_CASES["small"], T=300, H=256, E=5, k=3, I=256)
    print("case MXFP4 T=300 E=5 k=3", flush=True)
    _parity(w, full=False)


def test_mx4_streamed_equals_whole_batch():
    """4 micro-batches through a 2-slot ring, dW deferred to the last call, against one call
    over the whole batch: every output bit-identical (256-row flush segments)."""
    mok = _mok()
    w = inputs.replace(MX4_CASES["imbalanced"], T=1024)
    x, dy, wr, b, w1, w2 = _case(w)
    whole = _run_whole(w, x, dy, wr, b, w1, w2, gemm=mok.MXFP4)
    st = _run_streamed(w, 4, 2, x, dy, wr, b, w1, w2, gemm=mok.MXFP4)
    np.testing.assert_array_equal(st["idx"], whole["idx"])
    for n in ("gate", "y", "dx", "dgate", "dw1", "dw2", "dwr"):
        a, c = st[n], whole[n]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c), n


def test_mx4_empty_batch_writes_zero_weight_gradients():
    mok = _mok()
    E, H, I = 4, 256, 256
    d = mok.Desc(0, H, E, 2, I, act=mok.BF16, gemm=mok.MXFP4)
    buf = mok.Buffers(d, DEV)
    q = mok.MxWeights(d, DEV)
    w1 = torch.randn(E, 2 * I, H, device=DEV).to(torch.bfloat16)
    w2 = torch.randn(E, H, I, device=DEV).to(torch.bfloat16)
    mok.weights_quantize(d, w1, w2, q)
    for t in (buf.dw1, buf.dw2, buf.dwr):
        t.fill_(float("nan"))
    x = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    wr = torch.randn(E, H, device=DEV).to(torch.bfloat16)
    mok.step(d, buf, x, wr, None, None, None, x, mxw=q)
    torch.cuda.synchronize()
    for t in (buf.dw1, buf.dw2, buf.dwr):
        assert torch.all(t == 0)


def test_mx4_step_quantisers_bit_exact():
    """As the MXFP8 quantiser test: x and dY rows in full; h, dGU and the flush's dO, h, dGU,
    x on the blocks whose bf16 inputs equal the oracle's (at least a quarter of them)."""
    mok = _mok()
    w = inputs.replace(MX4_CASES["imbalanced"], T=512, H=256, E=8, k=2, I=256)
    M = 2
    x, dy, wr, b, w1, w2 = _case(w)
    Tm = w.T // M
    d = mok.Desc(Tm, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.MXFP4, mb_count=M, ring=M)
    st = mok.StreamedStep(d, DEV)
    q = mok.MxWeights(d, DEV)
    mok.weights_quantize(d, w1.to(DEV), w2.to(DEV), q)
    st.run(x.to(DEV), wr.to(DEV), b.to(DEV), q, dy.to(DEV))
    torch.cuda.synchronize()
    L = mok.mx_layout_query(d)
    idx, g, f, bw = _oracle(w, x, dy, wr, b, w1, w2, fmt="e2m1")
    np.testing.assert_array_equal(st.idx.cpu().numpy(), idx)
    H, I, k, E = w.H, w.I, w.k, w.E
    R = Tm * k
    xs, dys = x.double().numpy(), dy.double().numpy()
    fw, bwk = st.fwd_ws, st.bwd_ws
    fracs = {}
    rows_e = {e: [] for e in range(E)}
    for m in range(M):
        sc = orc.schedule(idx[m * Tm:(m + 1) * Tm], E, 32)
        gslot = m * R + sc["perm"]
        fo, bo = m * L["fwd_slot"], m * L["bwd_slot"]
        xq = _decode_e2m1(fw[fo + L["xq"]: fo + L["xq"] + Tm * H // 2]).reshape(Tm, H)
        el, s = orc.mx.mx_quantize(xs[m * Tm:(m + 1) * Tm], -1, "e2m1")
        np.testing.assert_array_equal(xq, el)
        np.testing.assert_array_equal(_kmaj(fw[fo + L["xs"]:], Tm, H // 32), s)
        dq = _decode_e2m1(bwk[bo + L["dyq"]: bo + L["dyq"] + Tm * H // 2]).reshape(Tm, H)
        el, s = orc.mx.mx_quantize(dys[m * Tm:(m + 1) * Tm], -1, "e2m1")
        np.testing.assert_array_equal(dq, el)
        np.testing.assert_array_equal(_kmaj(bwk[bo + L["dys"]:], Tm, H // 32), s)
        hg = mok.saved_layout_query(d)["h_offset"]
        h_gpu = _bf16_rows(st.saved[m], hg, R, I)
        hq = _decode_e2m1(fw[fo + L["hq"]: fo + L["hq"] + R * I // 2]).reshape(R, I)
        fracs["h%d" % m] = _compare_blocks("hq", hq, _kmaj(fw[fo + L["hs"]:], R, I // 32), f["h"][gslot], h_gpu,
                                           fmt="e2m1")
        dgu_gpu = _bf16_rows(bwk, L["st_dgu"] + 2 * m * R * 2 * I, R, 2 * I)
        gq = _decode_e2m1(bwk[bo + L["dguq"]: bo + L["dguq"] + R * I]).reshape(R, 2 * I)
        fracs["dgu%d" % m] = _compare_blocks("dguq", gq, _kmaj(bwk[bo + L["dgus"]:], R, 2 * I // 32),
                                             bw["dgu"][gslot], dgu_gpu, fmt="e2m1")
        for e in range(E):
            for r in range(sc["offsets"][e], sc["offsets"][e + 1]):
                rows_e[e].append((m * R + r, gslot[r]))
    K = L["kmax"]
    pofs = bwk[L["pofs"]: L["pofs"] + 4 * (E + 1)].view(torch.int32).cpu().numpy()
    gflat = g.ravel()
    ops = {
        "dO": ("dot", "dots", H, L["st_dos"], lambda s_: orc.bf16_round(gflat[s_][:, None] * dys[s_ // k])),
        "h": ("ht", "hts", I, L["st_h"], lambda s_: f["h"][s_]),
        "dGU": ("dgut", "dguts", 2 * I, L["st_dgu"], lambda s_: bw["dgu"][s_]),
        "x": ("xt", "xts", H, L["st_xs"], lambda s_: xs[s_ // k]),
    }
    for name, (qn, sn, F, so, ref_fn) in ops.items():
        qall = _decode_e2m1(bwk[L[qn]: L[qn] + F * K // 2]).reshape(F, K)
        sall = _kmaj(bwk[L[sn]:], F, K // 32)
        stash = _bf16_rows(bwk, so, M * R, F)
        tot = 0
        for e in range(E):
            n = len(rows_e[e])
            pad = pofs[e + 1] - pofs[e]
            assert pad == -(-n // 256) * 256, (e, n, pad)
            if n == 0:
                continue
            st_rows = np.array([r for r, _ in rows_e[e]])
            slots = np.array([s_ for _, s_ in rows_e[e]])
            ref = np.zeros((pad, F))
            gate_v = np.zeros((pad, F))
            ref[:n] = ref_fn(slots)
            gate_v[:n] = stash[st_rows]
            p0 = pofs[e]
            tot += _compare_blocks(name + "[%d]" % e, qall[:, p0:p0 + pad].T, sall[:, p0 // 32:(p0 + pad) // 32].T,
                                   ref, gate_v, axis_rows=True, fmt="e2m1")
        fracs[name] = tot
    print("blocks compared:", {k_: "%.3f" % v for k_, v in fracs.items()}, flush=True)


def test_mx4_wgrad_f32():
    """MXFP4 with MOK_FLAG_WGRAD_F32: fp32 weight gradients (one output tile per workgroup)
    and fp32 dWr, against the oracle's MXFP4 step with dW kept in fp32."""
    mok = _mok()
    w = inputs.replace(MX4_CASES["imbalanced"], T=512, H=256, E=8, k=2, I=256)
    x, dy, wr, b, w1, w2 = _case(w)
    g = _run_whole(w, x, dy, wr, b, w1, w2, wgrad_f32=True, gemm=mok.MXFP4)
    assert g["dw1"].dtype == torch.float32 and g["dwr"].dtype == torch.float32
    idx, gate, f, bw = _oracle(w, x, dy, wr, b, w1, w2, wfmt="f32", fmt="e2m1")
    np.testing.assert_array_equal(g["idx"], idx)
    errs = {"dw1": rel_fro(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
            "dw2": rel_fro(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
            "dwr": rel_fro(np64(g["dwr"]), bw["dwr"]), "dx": rel_fro(np64(g["dx"]), bw["dx"])}
    print("rel. Frobenius:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL_MX4, (k, v)


def test_mx4_grids_and_replay_bit_identical():
    """Persistent grids of 1, 7 and 300 workgroups, and forward-activation replay, give the
    streamed MXFP4 step's bits (4 micro-batches, 2-slot ring)."""
    mok = _mok()
    w = inputs.replace(MX4_CASES["imbalanced"], T=1024)
    case = _case(w)
    ref = _run_streamed(w, 4, 2, *case, gemm=mok.MXFP4)
    runs = [("grid %d" % g, dict(grid=g)) for g in (1, 7, 300)] + [("replay", dict(flags=mok.FLAG_REPLAY))]
    for label, kw in runs:
        print("case MXFP4 streamed 4x,", label, flush=True)
        got = _run_streamed(w, 4, 2, *case, gemm=mok.MXFP4, **kw)
        for n in ref:
            a, c = got[n], ref[n]
            same = np.array_equal(a, c) if isinstance(a, np.ndarray) else torch.equal(a, c)
            assert same, (label, n)
