"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Integer results (routing indices, logits, counts, offsets, permutation, tiles)
must match bit for bit; floating results within the relative Frobenius error
of the storage format (bf16 5e-3, fp32 1e-5) against the oracle, which
accumulates in fp64 and rounds at the same storage points.
"""
import numpy as np
import pytest
import torch

from harness import ROW_TOL, TOL, Case, np64, rel_fro, rel_fro_rows, run_gpu, run_oracle
from mixture_experts_layer_stable_amd import inputs

pytestmark = pytest.mark.gpu

SMALL = ["tiny_fp32", "small_bf16", "imbalanced_bf16"]


def _w(name, **kw):
    w = inputs.WORKLOADS[name]
    return inputs.replace(w, **kw) if kw else w


def _check_routing(g, o):
    np.testing.assert_array_equal(g["logits"], o["z"])
    np.testing.assert_array_equal(g["idx"], o["idx"])
    assert rel_fro(g["gate"], o["gate"]) <= 1e-6
    sc = o["sched"]
    np.testing.assert_array_equal(g["counts"], sc["counts"])
    np.testing.assert_array_equal(g["offsets"], sc["offsets"])
    np.testing.assert_array_equal(g["perm"], sc["perm"])
    np.testing.assert_array_equal(g["inv"], sc["inv"])
    assert g["num_tiles"] == len(sc["tiles"])
    np.testing.assert_array_equal(g["tiles"][: g["num_tiles"], :3], sc["tiles"])
    np.testing.assert_array_equal(g["tile_start"][-1], len(sc["tiles"]))


def _check_rows(pairs, row_tol):
    """Every row of every output within row_tol (see harness.ROW_TOL)."""
    rows = {n: rel_fro_rows(np64(a), r) for n, (a, r) in pairs.items()}
    for n, e in rows.items():
        assert e <= row_tol, ("row", n, e, rows)


def _check_forward(w, g, o, tol):
    fwd = o["fwd"]
    perm = o["sched"]["perm"]
    pairs = {"y": (g["y"], fwd["y"]), "a": (g["a"], fwd["a"][perm]), "u": (g["u"], fwd["u"][perm]),
             "h": (g["h"], fwd["h"][perm])}
    errs = {n: rel_fro(np64(a), r) for n, (a, r) in pairs.items()}
    for n, e in errs.items():
        assert e <= tol, (n, e, errs)
    _check_rows(pairs, ROW_TOL[w.act] if tol == TOL[w.act] else 4 * tol)
    return errs


def _check_backward(w, g, o, tol, router=True):
    b = o["bwd"]
    dw1 = np.stack([b["dw1"][e] for e in range(w.E)])
    dw2 = np.stack([b["dw2"][e] for e in range(w.E)])
    errs = {"dx": rel_fro(np64(g["dx"]), b["dx"]),
            "dw1": rel_fro(np64(g["dw1"]), dw1),
            "dw2": rel_fro(np64(g["dw2"]), dw2),
            "dgate": rel_fro(g["dgate"], b["dgate"])}
    pairs = {"dx": (g["dx"], b["dx"]), "dw1": (g["dw1"], dw1), "dw2": (g["dw2"], dw2)}
    if router:
        errs["dwr"] = rel_fro(np64(g["dwr"]), b["dwr"])
        pairs["dwr"] = (g["dwr"], b["dwr"])
    for n, e in errs.items():
        assert e <= tol, (n, e, errs)
    _check_rows(pairs, ROW_TOL[w.act] if tol == TOL[w.act] else 4 * tol)
    return errs


def _full(w, case=None, tol=None, **kw):
    case = case or Case(w)
    g = run_gpu(case, backward=w.backward or kw.pop("backward", False), **kw)
    o = run_oracle(case, backward="dx" in g, BM=g["tile_m"])
    _check_routing(g, o)
    tol = TOL[w.act] if tol is None else tol
    _check_forward(w, g, o, tol)
    if "dx" in g:
        _check_backward(w, g, o, tol)
    return g, o


@pytest.mark.parametrize("name", SMALL)
def test_workload_parity(name):
    """Every small workload end to end: routing bit-exact, forward (and backward) within tolerance."""
    w = inputs.WORKLOADS[name]
    print("case", name, flush=True)
    _full(w)


def test_tiny_fp32_backward_parity():
    """The fp32 path also runs the backward (the tiny workload's step is forward-only)."""
    w = _w("tiny_fp32", backward=True)
    _full(w)


@pytest.mark.parametrize("T,E", [(3000, 72), (5000, 72), (9000, 72), (17000, 72), (1000, 20), (3000, 20),
                                 (9000, 6), (777, 13)])
def test_route_token_group_sizes(T, E):
    """The router picks 4, 8, 16 or 32 tokens per workgroup by batch size (3000, 5000, 9000
    and 17000 tokens select each of them on 256 compute units for 72 experts; the last group
    is ragged); with at most 32 experts a wave holds tokens x experts, one or two chains per
    lane (1000 / 3000 tokens of 20 experts, 9000 of 6, a ragged 777 of 13): logits and
    indices equal the oracle's bit for bit, gates within 1e-6."""
    import oracle as orc
    from mixture_experts_layer_stable_amd import mok

    w = _w("imbalanced_bf16", T=T, E=E, k=3, H=256, I=128)
    print("case T=%d E=%d k=%d H=%d" % (w.T, w.E, w.k, w.H), flush=True)
    x, wr, b = inputs.make_x(w), inputs.make_wr(w), inputs.make_bias(w)
    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16)
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    logits = torch.empty(w.T, w.E, dtype=torch.float32, device="cuda")
    mok.route(d, x.cuda(), wr.cuda(), None if b is None else b.cuda(), idx, gate, logits)
    torch.cuda.synchronize()
    z, oi, og = orc.route(x.float().numpy(), wr.float().numpy(), w.k, None if b is None else b.numpy())
    np.testing.assert_array_equal(logits.cpu().numpy(), z)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    assert rel_fro(gate.cpu().double().numpy(), og) <= 1e-6


@pytest.mark.parametrize("T,E,k,H,I", [(77, 5, 2, 128, 128), (130, 100, 3, 256, 384), (40, 600, 4, 128, 128),
                                       (33, 8, 8, 128, 256), (50, 1, 1, 128, 128), (96, 40, 3, 384, 256),
                                       (64, 64, 2, 2048, 128), (256, 16, 2, 4096, 128)])
def test_ragged_and_odd_shapes(T, E, k, H, I):
    """Token counts that are not tile multiples, E not a multiple of 64, E > 512, k = E, E = 1;
    H = 384 (six 64-h chunks: a partial group of the small-batch router's 4-chunk Wr
    prefetch), H = 2048 (the largest H whose x rows that router stages whole) and H = 4096
    (above 2048 the router backward's dWr uses its 32-lane x 8-vector shape)."""
    w = _w("small_bf16", T=T, E=E, k=k, H=H, I=I)
    print("case", w, flush=True)
    _full(w)


def test_all_tokens_one_expert():
    """Worst-case imbalance: a +100 bias makes expert 3 every token's first choice (many tiles of
    one expert); experts never chosen must get zero weight gradients."""
    w = _w("small_bf16", T=300, E=16, k=2, H=128, I=128)
    bias = torch.zeros(16, dtype=torch.float32)
    bias[3] = 100.0
    bias[10:] = -100.0
    g, o = _full(w, Case(w, bias=bias))
    assert g["counts"][3] == 300
    assert np.all(g["counts"][10:] == 0)
    assert np.all(np64(g["dw1"][10:]) == 0) and np.all(np64(g["dw2"][10:]) == 0)
    assert np.all(np64(g["dwr"][10:]) == 0)


def test_zero_tokens_and_duplicate_router_rows():
    """x_t = 0 rows route to experts 0..k-1 with gates exactly 1/k; duplicated router rows tie and
    the lower expert index wins."""
    w = _w("small_bf16", T=64, E=8, k=2, H=128, I=128)
    case = Case(w)
    case.x[:10] = 0
    case.wr[5] = case.wr[2]
    g, o = _full(w, case)
    np.testing.assert_array_equal(g["idx"][:10], np.tile([0, 1], (10, 1)))
    assert np.all(g["gate"][:10] == 0.5)


def test_empty_batch():
    """T = 0: nothing to route; weight gradients are written as zeros."""
    from mixture_experts_layer_stable_amd import mok
    d = mok.Desc(0, 128, 4, 2, 128, act=mok.BF16)
    buf = mok.Buffers(d, "cuda")
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    wr = torch.randn(4, 128, device="cuda").to(torch.bfloat16)
    w1 = torch.randn(4, 256, 128, device="cuda").to(torch.bfloat16)
    w2 = torch.randn(4, 128, 128, device="cuda").to(torch.bfloat16)
    buf.dw1.fill_(1.0)
    buf.dw2.fill_(1.0)
    buf.dwr.fill_(1.0)
    mok.step(d, buf, x, wr, None, w1, w2, dy=torch.empty(0, 128, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(buf.dw1 == 0) and torch.all(buf.dw2 == 0) and torch.all(buf.dwr == 0)
    sv = buf.schedule_views()
    assert int(sv["num_tiles"][0]) == 0 and torch.all(sv["counts"] == 0)


def test_no_router_backward():
    """wr = dwr = NULL skips the router backward: dx is the expert term only."""
    w = _w("small_bf16", T=96, E=8, k=2, H=128, I=256)
    case = Case(w)
    g = run_gpu(case, router_grad=False)
    o = run_oracle(case, BM=g["tile_m"], router_grad=False)
    _check_routing(g, o)
    _check_backward(w, g, o, TOL["bf16"], router=False)


@pytest.mark.parametrize("H,I", [(128, 128), (256, 256)])
def test_wgrad_f32_flag(H, I):
    """MOK_FLAG_WGRAD_F32 writes dW1/dW2/dWr in fp32 (compared to the fp64 oracle rounded to fp32);
    H = I = 256 takes the 256 x 256 fp32-output weight-gradient tiles."""
    w = _w("small_bf16", T=128, E=8, k=2, H=H, I=I)
    case = Case(w)
    g = run_gpu(case, wgrad_f32=True)
    assert g["dw1"].dtype == torch.float32
    o = run_oracle(case, BM=g["tile_m"], wfmt="f32")
    b = o["bwd"]
    assert rel_fro(np64(g["dw1"]), np.stack([b["dw1"][e] for e in range(8)])) <= 5e-3
    assert rel_fro(np64(g["dwr"]), b["dwr"]) <= 5e-3


@pytest.mark.parametrize("name", ["small_bf16", "imbalanced_bf16"])
def test_bit_reproducible_across_runs_tiles_and_grids(name):
    """Two runs give identical bits; so do other schedule tile heights and persistent grid sizes
    (every output element is summed in an order that does not depend on either)."""
    w = inputs.WORKLOADS[name]
    case = Case(w)
    ref = run_gpu(case)
    variants = [dict(), dict(tile_m=128), dict(tile_m=64, grid=7), dict(grid=300), dict(tile_m=32, grid=1)]
    for kw in variants:
        g = run_gpu(case, **kw)
        for key in ("idx", "logits", "gate", "counts", "offsets", "perm", "inv", "dgate"):
            np.testing.assert_array_equal(g[key], ref[key], err_msg=str((kw, key)))
        for key in ("y", "a", "u", "h", "dx", "dw1", "dw2", "dwr"):
            assert torch.equal(g[key].view(torch.int16) if g[key].dtype == torch.bfloat16 else g[key],
                               ref[key].view(torch.int16) if ref[key].dtype == torch.bfloat16 else ref[key]), (kw, key)


@pytest.mark.parametrize("gemm", ["bf16", "mxfp8"])
def test_dw_tile_queues_reset_between_launches(gemm):
    """Weight-gradient launches with a few tiles per workgroup (here: 2048 tokens, Zipf
    routing) hand their tiles out from counters in the schedule header (lines 38-45 of 128
    bytes; word 0 counts tiles handed out, word 1 workgroups done), which each launch's
    last workgroup zeroes again. Three backwards in a row on the same buffers, each with
    another dY and its outputs pre-filled with NaN, equal one-shot runs on fresh buffers
    bit for bit, and the counters read zero after each."""
    from mixture_experts_layer_stable_amd import mok
    w = inputs.WORKLOADS["imbalanced_bf16"]
    dev = "cuda"
    x, wr, dy0 = inputs.make_x(w).to(dev), inputs.make_wr(w).to(dev), inputs.make_dy(w).to(dev)
    b = inputs.make_bias(w)
    b = None if b is None else b.to(dev)
    w1 = torch.stack([inputs.make_w1(w, e) for e in range(w.E)]).to(dev)
    w2 = torch.stack([inputs.make_w2(w, e) for e in range(w.E)]).to(dev)
    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.MXFP8 if gemm == "mxfp8" else mok.BF16)
    q = None
    if gemm == "mxfp8":
        q = mok.MxWeights(d, dev)
        mok.weights_quantize(d, w1, w2, q)
    names = ("y", "dx", "dgate", "dw1", "dw2", "dwr")

    def run(buf, dy):
        for n in names:
            getattr(buf, n).fill_(float("nan"))
        mok.step(d, buf, x, wr, b, None if q else w1, None if q else w2, dy, mxw=q)
        torch.cuda.synchronize()
        mok.check_schedule(d, buf.sched, "step")
        lines = buf.sched[38 * 128: 46 * 128].view(torch.int32).view(8, 32)[:, :2]
        assert torch.all(lines == 0), lines.cpu()
        return {n: getattr(buf, n).clone() for n in names}

    same = mok.Buffers(d, dev)
    for j in range(3):
        dy = torch.roll(dy0, 7 * j, 0)
        print("case", gemm, "backward", j, flush=True)
        got = run(same, dy)
        ref = run(mok.Buffers(d, dev), dy)
        for n in names:
            a, c = got[n], ref[n]
            assert not torch.isnan(a.float()).any(), (j, n)
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               c.view(torch.int16) if c.dtype == torch.bfloat16 else c), (j, n)


def test_default_tile_height_rule():
    """tile_m = 0 takes the tallest of 128/64/32 rows for which the FC1 GEMM has at least two
    tiles per compute unit even with every row packed into full tiles ((R / BM) * (2I / 256)
    >= 2 CUs: the pages' two full waves); MOK_FLAG_FUSED keeps 32 rows; an explicit tile_m is
    kept."""
    from mixture_experts_layer_stable_amd import mok
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def rule(R, I):
        for bm in (128, 64, 32):
            if (R // bm) * (2 * I // 256) >= 2 * cus:
                return bm
        return 32

    for T, E, k, H, I in ((2048, 32, 2, 1024, 512), (16384, 384, 8, 7168, 2048), (2048, 384, 8, 7168, 2048),
                          (64, 8, 2, 128, 256), (1024, 16, 2, 256, 512)):
        d = mok.Desc(T, H, E, k, I, act=mok.BF16)
        assert mok.schedule_layout_query(d)["tile_m"] == rule(T * k, I), (T, E, k, H, I)
        assert mok.schedule_layout_query(mok.Desc(T, H, E, k, I, act=mok.BF16, flags=mok.FLAG_FUSED))["tile_m"] == 32
        assert mok.schedule_layout_query(mok.Desc(T, H, E, k, I, act=mok.BF16, tile_m=128))["tile_m"] == 128
    if cus == 256:  # MI355X: the 2048-token workloads take 32-row tiles, the Kimi-K2 shapes 128
        assert mok.schedule_layout_query(mok.Desc(2048, 1024, 32, 2, 512, act=mok.BF16))["tile_m"] == 32
        assert mok.schedule_layout_query(mok.Desc(16384, 7168, 384, 8, 2048, act=mok.BF16))["tile_m"] == 128


def test_schedule_built_for_another_descriptor_is_rejected():
    """A schedule built for one descriptor and handed to forward/backward with another: every
    kernel checks the header's descriptor hash first, so nothing is written (outputs keep
    their sentinel) and the header's status word reads MOK_ERR_SCHEDULE_MISMATCH. Building
    the schedule for the right descriptor clears it."""
    from mixture_experts_layer_stable_amd import mok
    w = _w("small_bf16", T=96, E=8, k=2, H=128, I=128)
    case = Case(w)
    dev = "cuda"
    d_b = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16)
    for d_a in (mok.Desc(w.T, w.H, 12, w.k, w.I, act=mok.BF16), mok.Desc(64, w.H, w.E, w.k, w.I, act=mok.BF16),
                mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16, tile_m=64)):
        print("case schedule for", d_a, flush=True)
        buf = mok.Buffers(d_b, dev)
        nb = max(mok.workspace_query(d_a)["sched"], mok.workspace_query(d_b)["sched"])
        buf.sched = torch.empty(nb, dtype=torch.uint8, device=dev)
        x, wr = case.x.to(dev), case.wr.to(dev)
        w1, w2, dy = case.w1.to(dev), case.w2.to(dev), case.dy.to(dev)
        mok.route(d_b, x, wr, None, buf.idx, buf.gate)
        idx_a = torch.zeros(d_a.T, d_a.k, dtype=torch.int32, device=dev)
        mok.schedule_build(d_a, idx_a, buf.sched)       # same buffer, other descriptor
        for t in (buf.y, buf.dx, buf.dw1, buf.dw2, buf.dwr):
            t.fill_(7.0)
        buf.dgate.fill_(7.0)
        mok.moe_forward(d_b, buf.sched, x, buf.gate, w1, w2, buf.y, buf.saved, buf.fwd_ws)
        mok.moe_backward(d_b, buf.sched, x, buf.idx, buf.gate, w1, w2, wr, buf.saved, dy, buf.dx, buf.dw1, buf.dw2,
                         buf.dgate, buf.dwr, buf.bwd_ws)
        torch.cuda.synchronize()
        assert mok.schedule_status(d_b, buf.sched) == mok.ERR_SCHEDULE_MISMATCH
        with pytest.raises(mok.MokError):
            mok.check_schedule(d_b, buf.sched)
        for t in (buf.y, buf.dx, buf.dw1, buf.dw2, buf.dwr, buf.dgate):
            assert torch.all(t == 7.0)
        mok.schedule_build(d_b, buf.idx, buf.sched)
        torch.cuda.synchronize()
        assert mok.schedule_status(d_b, buf.sched) == 0


@pytest.mark.parametrize("name,kw", [("small_bf16", {}), ("imbalanced_bf16", dict(T=600, E=12, k=3)),
                                     ("tiny_fp32", dict(backward=True))])
def test_replay_bit_identical(name, kw):
    """Forward-activation replay (MOK_FLAG_REPLAY): the forward keeps no activations and the
    backward forms a, u, h again with the forward's FC1; every output equals the stored
    path's bit for bit."""
    from mixture_experts_layer_stable_amd import mok
    w = _w(name, **kw)
    case = Case(w)
    ref = run_gpu(case, backward=True)
    got = run_gpu(case, backward=True, replay=True)
    for key in ("idx", "gate", "perm", "dgate"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    for key in ("y", "dx", "dw1", "dw2", "dwr"):
        a, b = got[key], ref[key]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), key


def _same(got, ref, keys):
    for key in keys:
        a, b = got[key], ref[key]
        if isinstance(a, np.ndarray):
            np.testing.assert_array_equal(a, b, err_msg=key)
        else:
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), key


@pytest.mark.parametrize("name,kw,grid", [("small_bf16", {}, 0), ("imbalanced_bf16", {}, 0),
                                          ("small_bf16", dict(T=300, E=12, k=3, H=256, I=128), 7),
                                          ("small_bf16", dict(T=256, E=16, k=2, H=4096, I=128), 0),
                                          ("small_bf16", dict(T=200, E=8, k=2, H=384, I=384), 300)])
def test_fused_persistent_kernels_bit_identical(name, kw, grid):
    """MOK_FLAG_FUSED: the forward and the backward each as one cooperative persistent launch
    with grid barriers between the stages; every output equals the separate kernels' bits
    (also with 7 workgroups and with a grid request above the compute-unit count, H = 4096
    and H, I not multiples of 256), and the oracle agrees within the bf16 tolerance."""
    w = _w(name, **kw)
    print("case fused", w, "grid", grid, flush=True)
    case = Case(w)
    ref = run_gpu(case)
    got = run_gpu(case, fused=True, grid=grid)
    assert got["tile_m"] == 32
    _same(got, ref, ("idx", "gate", "perm", "dgate", "y", "a", "u", "h", "dx", "dw1", "dw2", "dwr"))
    o = run_oracle(case, BM=32)
    _check_forward(w, got, o, TOL["bf16"])
    _check_backward(w, got, o, TOL["bf16"])


def test_fused_replay_and_no_router_backward():
    """Fused kernels with activation replay (a separate FC1 launch before the fused backward)
    and with the router backward skipped (wr = dwr = NULL)."""
    w = _w("small_bf16", T=512, E=16)
    case = Case(w)
    _same(run_gpu(case, fused=True, replay=True), run_gpu(case), ("y", "dx", "dw1", "dw2", "dwr", "dgate"))
    _same(run_gpu(case, fused=True, router_grad=False), run_gpu(case, router_grad=False),
          ("y", "dx", "dw1", "dw2", "dgate"))


def test_fused_needs_bf16_and_32_row_tiles():
    from mixture_experts_layer_stable_amd import mok
    w = _w("small_bf16", T=256, E=8, H=256, I=256)
    case = Case(w)
    with pytest.raises(mok.MokError) as ei:
        run_gpu(case, fused=True, tile_m=64)
    assert ei.value.status == 3
    with pytest.raises(mok.MokError) as ei:
        run_gpu(Case(_w("tiny_fp32", backward=True)), fused=True)
    assert ei.value.status == 4
    # k * I/32 = 4096 d-gate partials per token exceed what one workgroup keeps in LDS
    with pytest.raises(mok.MokError) as ei:
        run_gpu(Case(_w("small_bf16", T=64, E=16, k=16, H=128, I=8192)), fused=True, tile_m=32)
    assert ei.value.status == 3
