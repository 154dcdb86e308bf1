"""GPU parity of the MXFP8 path (E4M3 elements, E8M0 scale per 32 along each GEMM's K).

* the weight quantisers (four orientations) against the oracle's quantiser, bit for bit,
  on weights with planted edge blocks (all zero, 2^+-40 magnitudes, saturation, ties);
* one MXFP8 layer step (route, schedule, forward, backward) against the oracle's MXFP8
  step, which quantises every GEMM operand at the same points: rel. Frobenius <= 2e-2;
* the streamed step (micro-batches through the ring, weight gradients deferred to the
  last backward call) bit-identical to one call over the whole batch;
* repeated steps, and persistent grids of 1, 7 and 300 workgroups, bit-identical; an
  empty batch still writes zero weight gradients.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from harness import np64, rel_fro, rel_fro_rows
from mixture_experts_layer_stable_amd import inputs

pytestmark = pytest.mark.gpu

TOL_MX = 2e-2
# every single row (last-axis vector) of an output: a row holds few elements and one
# quantisation decision taken differently at a near-tie (fp32 against the oracle's fp64
# inputs to a quantiser) moves it by up to an element step; largest measured 7.4e-2
ROW_TOL_MX = 0.15
DEV = "cuda"


def _mok():
    from mixture_experts_layer_stable_amd import mok
    return mok


def _decode_e4m3(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.float8_e4m3fn).double().numpy()


def _edge_weights(E, rows, cols, seed):
    """bf16 weights with random per-block magnitudes and planted special blocks."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((E, rows, cols)) * np.exp2(rng.integers(-40, 41, (E, rows // 32, 1, cols // 32, 1))
                                                      ).repeat(32, 2).repeat(32, 4).reshape(E, rows, cols)
    w[0, :32, :32] = 0.0                                  # all-zero block (both orientations)
    w[0, 32:64, :] *= 2.0**-120                           # tiny: scale clamps at 2^-127
    w[-1, -32:, -32:] = 1.9 * 2.0**10                     # 1.9 * 2^10: elements 1.9 * 2^8 -> saturate to 448
    w[-1, -1, -1] = 2.0**10                               # block max sets the scale
    w[1, 5, :] = 2.0**-9 * 3 * (1 + (np.arange(cols) % 2))  # subnormal ties under a large block max
    return torch.from_numpy(w).to(torch.bfloat16)


def test_weights_quantize_bit_exact():
    mok = _mok()
    E, H, I = 3, 256, 128
    d = mok.Desc(64, H, E, 2, I, act=mok.BF16, gemm=mok.MXFP8)
    w1 = _edge_weights(E, 2 * I, H, 1)
    w2 = _edge_weights(E, H, I, 2)
    q = mok.MxWeights(d, DEV)
    mok.weights_quantize(d, w1.to(DEV), w2.to(DEV), q)
    torch.cuda.synchronize()
    W1 = w1.double().numpy()
    W2 = w2.double().numpy()
    cases = {
        "w1": (q.w1q, q.w1s, W1, -1),                                  # [E][2I][H] along H
        "w2": (q.w2q, q.w2s, W2, -1),                                  # [E][H][I] along I
        "w2t": (q.w2tq, q.w2ts, np.swapaxes(W2, 1, 2), -1),            # [E][I][H] along H
        "w1t": (q.w1tq, q.w1ts, np.swapaxes(W1, 1, 2), -1),            # [E][H][2I] along 2I
    }
    for name, (tq, ts, ref, ax) in cases.items():
        el, s = orc.mx.mx_quantize(ref, ax)
        # stored K-tile-major [E][K/128][rows][4] -> [E][rows][K/32]
        kt = ts.cpu().numpy().astype(np.int64)
        got_s = np.ascontiguousarray(kt.transpose(0, 2, 1, 3)).reshape(s.shape) - 127
        np.testing.assert_array_equal(got_s, s, err_msg=name + " scales")
        np.testing.assert_array_equal(_decode_e4m3(tq), el, err_msg=name + " elements")


# ---------------------------------------------------------------------------------------

def _case(w):
    x = inputs.make_x(w)
    dy = inputs.make_dy(w)
    wr = inputs.make_wr(w)
    b = inputs.make_bias(w)
    w1 = torch.stack([inputs.make_w1(w, e) for e in range(w.E)])
    w2 = torch.stack([inputs.make_w2(w, e) for e in range(w.E)])
    return x, dy, wr, b, w1, w2


def _run_whole(w, x, dy, wr, b, w1, w2, tile_m=0, router_grad=True, wgrad_f32=False, gemm=None):
    mok = _mok()
    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.MXFP8 if gemm is None else gemm, tile_m=tile_m,
                 flags=mok.FLAG_WGRAD_F32 if wgrad_f32 else 0)
    buf = mok.Buffers(d, DEV, wgrad_f32=wgrad_f32)
    q = mok.MxWeights(d, DEV)
    w1d, w2d = w1.to(DEV), w2.to(DEV)
    mok.weights_quantize(d, w1d, w2d, q)
    xd, dyd, wrd = x.to(DEV), dy.to(DEV), wr.to(DEV)
    bd = None if b is None else b.to(DEV)
    mok.step(d, buf, xd, wrd, bd, None, None, dyd, router_grad=router_grad, mxw=q)
    torch.cuda.synchronize()
    mok.check_schedule(d, buf.sched, "MXFP8 step")
    out = dict(idx=buf.idx.cpu().numpy(), gate=buf.gate.cpu(), y=buf.y.cpu(), dx=buf.dx.cpu(),
               dgate=buf.dgate.cpu(), dw1=buf.dw1.cpu(), dw2=buf.dw2.cpu(), perm=buf.schedule_views()["perm"].cpu())
    if router_grad:
        out["dwr"] = buf.dwr.cpu()
    sv = buf.saved_views()
    out.update(a=sv["a"].cpu(), u=sv["u"].cpu(), h=sv["h"].cpu())
    return out


def _run_streamed(w, M, ring, x, dy, wr, b, w1, w2, tile_m=0, grid=0, flags=0, gemm=None):
    mok = _mok()
    d = mok.Desc(w.T // M, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.MXFP8 if gemm is None else gemm,
                 tile_m=tile_m, mb_count=M, ring=ring, grid=grid, flags=flags)
    st = mok.StreamedStep(d, DEV)
    q = mok.MxWeights(d, DEV)
    mok.weights_quantize(d, w1.to(DEV), w2.to(DEV), q)
    st.run(x.to(DEV), wr.to(DEV), None if b is None else b.to(DEV), q, dy.to(DEV))
    torch.cuda.synchronize()
    return dict(idx=st.idx.cpu().numpy(), gate=st.gate.cpu(), y=st.y.cpu(), dx=st.dx.cpu(), dgate=st.dgate.cpu(),
                dw1=st.dw1.cpu(), dw2=st.dw2.cpu(), dwr=st.dwr.cpu())


def _oracle(w, x, dy, wr, b, w1, w2, wfmt="bf16", fmt="e4m3"):
    xs, dys, wrs = x.float().numpy(), dy.float().numpy(), wr.float().numpy()
    z, idx, g = orc.route(xs, wrs, w.k, None if b is None else b.numpy())
    W = orc.DenseWeights(w1.float().numpy(), w2.float().numpy())
    f = orc.mx.forward_mx(xs, W, idx, g, w.E, w.I, fmt=fmt)
    bw = orc.mx.backward_mx(xs, W, wrs, idx, g, f, dys, w.I, wfmt=wfmt, fmt=fmt)
    return idx, g, f, bw


MX_CASES = {
    "small": inputs.replace(inputs.WORKLOADS["small_bf16"], gemm="mxfp8"),
    "imbalanced": inputs.replace(inputs.WORKLOADS["imbalanced_bf16"], gemm="mxfp8"),
}


@pytest.mark.parametrize("name,tile_m", [("small", 0), ("imbalanced", 0), ("imbalanced", 32), ("small", 64)])
def test_mx_step_parity(name, tile_m):
    w = MX_CASES[name]
    print("case", name, "tile_m", tile_m, flush=True)
    x, dy, wr, b, w1, w2 = _case(w)
    g = _run_whole(w, x, dy, wr, b, w1, w2, tile_m=tile_m)
    idx, gate, f, bw = _oracle(w, x, dy, wr, b, w1, w2)
    np.testing.assert_array_equal(g["idx"], idx)
    perm = g["perm"].numpy()
    errs = {
        "gate": rel_fro(g["gate"].numpy(), gate),
        "y": rel_fro(np64(g["y"]), f["y"]),
        "a": rel_fro(np64(g["a"]), f["a"][perm]),
        "u": rel_fro(np64(g["u"]), f["u"][perm]),
        "h": rel_fro(np64(g["h"]), f["h"][perm]),
        "dx": rel_fro(np64(g["dx"]), bw["dx"]),
        "dgate": rel_fro(g["dgate"].numpy(), bw["dgate"]),
        "dw1": rel_fro(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
        "dw2": rel_fro(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
        "dwr": rel_fro(np64(g["dwr"]), bw["dwr"]),
    }
    print("rel. Frobenius:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL_MX, (k, v)
    rows = {
        "y": rel_fro_rows(np64(g["y"]), f["y"]),
        "h": rel_fro_rows(np64(g["h"]), f["h"][perm]),
        "dx": rel_fro_rows(np64(g["dx"]), bw["dx"]),
        "dw1": rel_fro_rows(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
        "dw2": rel_fro_rows(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
        "dwr": rel_fro_rows(np64(g["dwr"]), bw["dwr"]),
    }
    print("largest row error:", {k: "%.2e" % v for k, v in rows.items()}, flush=True)
    for k, v in rows.items():
        assert v <= ROW_TOL_MX, ("row", k, v)


def test_mx_streamed_equals_whole_batch():
    """4 micro-batches through a 2-slot ring, backward 3..0 with dW deferred, against
    one call over all 2048 tokens: every output bit-identical."""
    w = MX_CASES["imbalanced"]
    x, dy, wr, b, w1, w2 = _case(w)
    whole = _run_whole(w, x, dy, wr, b, w1, w2, tile_m=64)
    st = _run_streamed(w, 4, 2, x, dy, wr, b, w1, w2, tile_m=64)
    np.testing.assert_array_equal(st["idx"], whole["idx"])
    for n in ("gate", "y", "dx", "dgate", "dw1", "dw2", "dwr"):
        a, c = st[n], whole[n]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c), n


def test_mx_grids_bit_identical():
    """Persistent grids of 1, 7 and 300 workgroups (the row GEMMs and the pipelined
    weight-gradient kernel walk their tiles in a different order and number of passes)
    give the same bits as the default one-per-CU grid."""
    w = MX_CASES["imbalanced"]
    case = _case(w)
    ref = _run_streamed(w, 4, 2, *case)
    for grid in (1, 7, 300):
        print("case imbalanced streamed 4x, grid", grid, flush=True)
        got = _run_streamed(w, 4, 2, *case, grid=grid)
        for n in ref:
            a, b = ref[n], got[n]
            same = np.array_equal(a, b) if isinstance(a, np.ndarray) else torch.equal(a, b)
            assert same, ("grid", grid, n)


def test_mx_repeat_bit_identical():
    w = inputs.replace(MX_CASES["small"], T=512)
    x, dy, wr, b, w1, w2 = _case(w)
    r1 = _run_whole(w, x, dy, wr, b, w1, w2)
    r2 = _run_whole(w, x, dy, wr, b, w1, w2)
    for n in ("y", "dx", "dgate", "dw1", "dw2", "dwr"):
        assert torch.equal(r1[n].view(torch.int16) if r1[n].dtype == torch.bfloat16 else r1[n],
                           r2[n].view(torch.int16) if r2[n].dtype == torch.bfloat16 else r2[n]), n


def test_mx_empty_batch_writes_zero_weight_gradients():
    mok = _mok()
    E, H, I = 4, 256, 128
    d = mok.Desc(0, H, E, 2, I, act=mok.BF16, gemm=mok.MXFP8)
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


def _mx_parity(w, tile_m=0):
    x, dy, wr, b, w1, w2 = _case(w)
    g = _run_whole(w, x, dy, wr, b, w1, w2, tile_m=tile_m)
    idx, gate, f, bw = _oracle(w, x, dy, wr, b, w1, w2)
    np.testing.assert_array_equal(g["idx"], idx)
    errs = {
        "y": rel_fro(np64(g["y"]), f["y"]),
        "dx": rel_fro(np64(g["dx"]), bw["dx"]),
        "dgate": rel_fro(g["dgate"].numpy(), bw["dgate"]),
        "dw1": rel_fro(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
        "dw2": rel_fro(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
        "dwr": rel_fro(np64(g["dwr"]), bw["dwr"]),
    }
    print("rel. Frobenius:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL_MX, (k, v)


@pytest.mark.parametrize("tile_m", [0, 32])
def test_mx_ragged_odd_shape(tile_m):
    """T = 300 tokens, k = 3 of E = 5 experts: segments that are not multiples of 32, 64 or
    128 rows, a token-block tail in every expert's weight-gradient operands."""
    w = inputs.replace(MX_CASES["small"], T=300, H=256, E=5, k=3, I=128)
    print("case T=300 E=5 k=3 tile_m", tile_m, flush=True)
    _mx_parity(w, tile_m)


def test_mx_single_expert_top1():
    """E = 1, k = 1: every token in one segment, gates exactly 1."""
    w = inputs.replace(MX_CASES["small"], T=200, H=256, E=1, k=1, I=256)
    _mx_parity(w)


def test_mx_streamed_three_slots_odd_count():
    """3 micro-batches through a 3-slot ring against one call over the whole batch."""
    w = inputs.replace(MX_CASES["imbalanced"], T=768)
    x, dy, wr, b, w1, w2 = _case(w)
    whole = _run_whole(w, x, dy, wr, b, w1, w2)
    st = _run_streamed(w, 3, 3, x, dy, wr, b, w1, w2)
    for n in ("y", "dx", "dgate", "dw1", "dw2", "dwr"):
        a, c = st[n], whole[n]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c), n


def test_mx_wgrad_f32():
    """MXFP8 with MOK_FLAG_WGRAD_F32: fp32 weight gradients (one output tile per workgroup) and
    the fp32 dWr sums, against the oracle's MXFP8 step with dW kept in fp32."""
    w = inputs.replace(MX_CASES["imbalanced"], T=512, H=256, E=8, k=2, I=256)
    x, dy, wr, b, w1, w2 = _case(w)
    g = _run_whole(w, x, dy, wr, b, w1, w2, wgrad_f32=True)
    assert g["dw1"].dtype == torch.float32 and g["dwr"].dtype == torch.float32
    idx, gate, f, bw = _oracle(w, x, dy, wr, b, w1, w2, wfmt="f32")
    np.testing.assert_array_equal(g["idx"], idx)
    errs = {"dw1": rel_fro(np64(g["dw1"]), np.stack([bw["dw1"][e] for e in range(w.E)])),
            "dw2": rel_fro(np64(g["dw2"]), np.stack([bw["dw2"][e] for e in range(w.E)])),
            "dwr": rel_fro(np64(g["dwr"]), bw["dwr"]), "dx": rel_fro(np64(g["dx"]), bw["dx"])}
    print("rel. Frobenius:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL_MX, (k, v)


# ---------------------------------------------------------------------------------------
# Bit-exact checks of the quantisers inside the step: the activation row quantisers (x, dY),
# the fc1 / dh epilogue quantisers (h, dGU) and the flush's token-axis quantisers (dO, h,
# dGU, x over each expert's rows of the step). Expected bytes are the oracle quantiser's
# encoding of the oracle's own bf16 values. Where a value is the result of a GEMM (h, dGU)
# or of a product with the fp32 gate (dO), the GPU's bf16 value can differ from the
# oracle's by one rounding step; a 32-element block is compared only where the GPU's stored
# bf16 inputs of that block equal the oracle's (the GPU values only select blocks, they are
# never an input of the expected bytes). Inputs (x, dY) are compared in full; for the GEMM
# results about half of the blocks match the oracle's bf16 values exactly (measured 53 %
# for h at K = 256), so at least a quarter of the blocks must be compared.

def _kmaj(s_u8: torch.Tensor, rows: int, kb: int) -> np.ndarray:
    """K-tile-major scale bytes [kb/4][rows][4] -> exponents [rows][kb]."""
    a = s_u8.cpu().numpy().astype(np.int64)[: kb * rows].reshape(kb // 4, rows, 4)
    return np.ascontiguousarray(a.transpose(1, 0, 2)).reshape(rows, kb) - 127


def _bf16_rows(buf: torch.Tensor, off: int, rows: int, cols: int) -> np.ndarray:
    return buf[off: off + 2 * rows * cols].cpu().view(torch.bfloat16).view(rows, cols).double().numpy()


def _compare_blocks(name, got_el, got_s, ref_vals, gate_vals, axis_rows=False, fmt="e4m3"):
    """got_el/got_s: decoded GPU elements and scale exponents; ref_vals: the oracle's bf16
    values (blocks of 32 along the last axis, or along axis 0 when axis_rows); gate_vals:
    the GPU's stored bf16 values of the same elements."""
    if axis_rows:
        got_el, ref_vals, gate_vals = got_el.T, ref_vals.T, gate_vals.T
        got_s = got_s.T
    el, s = orc.mx.mx_quantize(ref_vals, -1, fmt)
    nb = ref_vals.shape[-1] // 32
    same = np.all((ref_vals == gate_vals).reshape(ref_vals.shape[:-1] + (nb, 32)), axis=-1)
    frac = same.mean()
    assert frac >= 0.25, (name, "blocks comparable", frac)
    np.testing.assert_array_equal(got_s[same], s[same], err_msg=name + " scales")
    bel = got_el.reshape(el.shape[:-1] + (nb, 32))[same]
    np.testing.assert_array_equal(bel, el.reshape(el.shape[:-1] + (nb, 32))[same], err_msg=name + " elements")
    return frac


def test_mx_step_quantisers_bit_exact():
    mok = _mok()
    w = inputs.replace(MX_CASES["imbalanced"], T=512, H=256, E=8, k=2, I=256)
    M = 2
    x, dy, wr, b, w1, w2 = _case(w)
    Tm = w.T // M
    d = mok.Desc(Tm, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.MXFP8, mb_count=M, ring=M)
    st = mok.StreamedStep(d, DEV)
    q = mok.MxWeights(d, DEV)
    mok.weights_quantize(d, w1.to(DEV), w2.to(DEV), q)
    st.run(x.to(DEV), wr.to(DEV), b.to(DEV), q, dy.to(DEV))
    torch.cuda.synchronize()
    L = mok.mx_layout_query(d)
    idx, g, f, bw = _oracle(w, x, dy, wr, b, w1, w2)
    np.testing.assert_array_equal(st.idx.cpu().numpy(), idx)
    H, I, k, E = w.H, w.I, w.k, w.E
    R = Tm * k
    xs, dys = x.double().numpy(), dy.double().numpy()
    fw, bwk = st.fwd_ws, st.bwd_ws
    fracs = {}
    rows_e = {e: [] for e in range(E)}           # (micro-batch, routed row, global slot) per expert
    for m in range(M):
        sc = orc.schedule(idx[m * Tm:(m + 1) * Tm], E, 32)
        gslot = m * R + sc["perm"]                # routed row -> global flat slot
        fo, bo = m * L["fwd_slot"], m * L["bwd_slot"]
        # x and dY rows (inputs: every block compared)
        xq = _decode_e4m3(fw[fo + L["xq"]: fo + L["xq"] + Tm * H]).reshape(Tm, H)
        el, s = orc.mx.mx_quantize(xs[m * Tm:(m + 1) * Tm], -1)
        np.testing.assert_array_equal(xq, el)
        np.testing.assert_array_equal(_kmaj(fw[fo + L["xs"]:], Tm, H // 32), s)
        dq = _decode_e4m3(bwk[bo + L["dyq"]: bo + L["dyq"] + Tm * H]).reshape(Tm, H)
        el, s = orc.mx.mx_quantize(dys[m * Tm:(m + 1) * Tm], -1)
        np.testing.assert_array_equal(dq, el)
        np.testing.assert_array_equal(_kmaj(bwk[bo + L["dys"]:], Tm, H // 32), s)
        # fc1 epilogue: h rows (routed order) along I
        hg = mok.saved_layout_query(d)["h_offset"]
        h_gpu = _bf16_rows(st.saved[m], hg, R, I)
        hq = _decode_e4m3(fw[fo + L["hq"]: fo + L["hq"] + R * I]).reshape(R, I)
        fracs["h%d" % m] = _compare_blocks("hq", hq, _kmaj(fw[fo + L["hs"]:], R, I // 32), f["h"][gslot], h_gpu)
        # dh epilogue: dGU rows along 2I (the GPU's bf16 dGU rows are in the stash)
        dgu_gpu = _bf16_rows(bwk, L["st_dgu"] + 2 * m * R * 2 * I, R, 2 * I)
        gq = _decode_e4m3(bwk[bo + L["dguq"]: bo + L["dguq"] + R * 2 * I]).reshape(R, 2 * I)
        fracs["dgu%d" % m] = _compare_blocks("dguq", gq, _kmaj(bwk[bo + L["dgus"]:], R, 2 * I // 32),
                                             bw["dgu"][gslot], dgu_gpu)
        for e in range(E):
            for r in range(sc["offsets"][e], sc["offsets"][e + 1]):
                rows_e[e].append((m * R + r, gslot[r]))
    # flush: token-axis operands over each expert's rows of the whole step, 128-padded segments
    K = L["kmax"]
    pofs = bwk[L["pofs"]: L["pofs"] + 4 * (E + 1)].view(torch.int32).cpu().numpy()
    gflat = g.ravel()
    ops = {  # name: (q, s, F, stash offset, oracle rows by global slot)
        "dO": ("dot", "dots", H, L["st_dos"], lambda s_: orc.bf16_round(gflat[s_][:, None] * dys[s_ // k])),
        "h": ("ht", "hts", I, L["st_h"], lambda s_: f["h"][s_]),
        "dGU": ("dgut", "dguts", 2 * I, L["st_dgu"], lambda s_: bw["dgu"][s_]),
        "x": ("xt", "xts", H, L["st_xs"], lambda s_: xs[s_ // k]),
    }
    for name, (qn, sn, F, so, ref_fn) in ops.items():
        qall = _decode_e4m3(bwk[L[qn]: L[qn] + F * K]).reshape(F, K)
        sall = _kmaj(bwk[L[sn]:], F, K // 32)                   # [F][K/32]
        stash = _bf16_rows(bwk, so, M * R, F)
        tot = 0
        for e in range(E):
            n = len(rows_e[e])
            pad = pofs[e + 1] - pofs[e]
            assert pad == -(-n // 128) * 128, (e, n, pad)
            if n == 0:
                continue
            st_rows = np.array([r for r, _ in rows_e[e]])
            slots = np.array([s_ for _, s_ in rows_e[e]])
            ref = np.zeros((pad, F))
            gate_v = np.zeros((pad, F))
            ref[:n] = ref_fn(slots)
            gate_v[:n] = stash[st_rows]
            p0 = pofs[e]
            fr = _compare_blocks(name + "[%d]" % e, qall[:, p0:p0 + pad].T, sall[:, p0 // 32:(p0 + pad) // 32].T,
                                 ref, gate_v, axis_rows=True)
            tot += fr
        fracs[name] = tot
    print("blocks compared:", {k_: "%.3f" % v for k_, v in fracs.items()}, flush=True)


def test_mx_replay_streamed_bit_identical():
    """Forward-activation replay with the streamed MXFP8 step (4 micro-batches, 2-slot ring):
    the backward of each micro-batch quantises x and runs FC1 again; every output equals the
    stored path's bit for bit."""
    mok = _mok()
    w = inputs.replace(MX_CASES["imbalanced"], T=1024)
    x, dy, wr, b, w1, w2 = _case(w)
    ref = _run_streamed(w, 4, 2, x, dy, wr, b, w1, w2)
    got = _run_streamed(w, 4, 2, x, dy, wr, b, w1, w2, flags=mok.FLAG_REPLAY)
    for n in ref:
        a, c = got[n], ref[n]
        same = np.array_equal(a, c) if isinstance(a, np.ndarray) else torch.equal(a, c)
        assert same, n
