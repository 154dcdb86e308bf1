"""Pins of the oracle's MXFP8 quantisation (OCP MX v1.0: E4M3 elements, E8M0 scale per
32-element block) and of its quantisation points in the layer step."""
import numpy as np
import pytest
import torch

import oracle as orc
from oracle import mx


def test_e4m3_rounding_matches_torch():
    """Library routine: torch's float8_e4m3fn conversion (round to nearest even, subnormals)."""
    rng = np.random.default_rng(0)
    v = rng.standard_normal(300000) * np.exp2(rng.uniform(-14, 8.8, 300000))
    v = np.clip(v, -448, 448).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(mx.e4m3_round(v), ref)


def test_mx_hand_examples():
    """Scale = floor(log2 amax) - 8; amax 1.0 -> element 256; saturation; zero block; ties."""
    blk = np.zeros(32)
    blk[0], blk[1], blk[2], blk[3] = 1.0, 0.9, 2.0**-18, 3 * 2.0**-18
    blk[4], blk[5] = 5 * 2.0**-18, 3 * 2.0**-19
    el, s = mx.mx_quantize(blk)
    assert s.tolist() == [-8]
    assert el[0] == 256.0                       # 1.0 / 2^-8
    assert el[1] == 224.0                       # 230.4 -> spacing 16 in [128, 256)
    assert el[2] == 0.0                         # 2^-10 = half a subnormal step: ties to even 0
    assert el[3] == 2 * 2.0**-9                 # 1.5 steps ties to even 2 steps
    assert el[4] == 2 * 2.0**-9                 # 2.5 steps ties to even 2 steps
    assert el[5] == 2.0**-9                     # 0.75 steps rounds to 1 step
    blk[0] = 1.9                                # 1.9 * 256 = 486.4 > 448 -> saturate
    el, s = mx.mx_quantize(blk)
    assert s.tolist() == [-8] and el[0] == 448.0
    el, s = mx.mx_quantize(np.zeros(64))
    assert s.tolist() == [-127, -127] and np.all(el == 0)
    el, s = mx.mx_quantize(np.full(32, -3.0 * 2.0**-100))
    assert s.tolist() == [-107] and np.all(el == -384.0)


def test_mx_idempotent_and_error_bound():
    """Quantising a quantised tensor changes nothing; elements below saturation are within
    half a step (relative 2^-4, absolute 2^(s-10) for subnormals) of the input."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((40, 256)) * np.exp2(rng.uniform(-8, 8, (40, 1)))
    q = mx.mx(v)
    np.testing.assert_array_equal(mx.mx(q), q)
    el, s = mx.mx_quantize(v)
    sc = np.repeat(np.exp2(s.astype(float)), 32, axis=1)
    ok = np.abs(v / sc) <= 448
    err = np.abs(q - v)
    assert np.all(err[ok] <= np.maximum(np.abs(v[ok]) * 2.0**-4, sc[ok] * 2.0**-10) * (1 + 1e-12))


def _exact_along(shape, axis, rng, spread=30):
    """Values exactly representable in MX blocks along `axis`: each element is a small
    integer / 8 times 2^m, with m constant along `axis` and varying by up to 2^spread
    across the other axis, so that blocking along the other axis flushes the small ones."""
    v = rng.integers(-7, 8, shape).astype(np.float64) / 8.0
    other = 1 - axis
    m = np.exp2(rng.integers(-spread, 1, shape[other]).astype(np.float64))
    return v * (m[:, None] if other == 0 else m[None, :])


def _step(x, dy, w1, w2, rng, E=3, k=2, I=64, fmt="e4m3"):
    wr = rng.standard_normal((E, x.shape[1])) * 0.2
    z, idx, g = orc.route(x, wr, k, exact=True)
    W = orc.DenseWeights(w1, w2)
    fm, fb = mx.forward_mx(x, W, idx, g, E, I, fmt=fmt), orc.forward(x, W, idx, g, "bf16", E, I)
    bm = mx.backward_mx(x, W, wr, idx, g, fm, dy, I, fmt=fmt)
    bb = orc.backward(x, W, wr, idx, g, fb, dy, "bf16", I)
    return idx, fm, fb, bm, bb


def _worst_rel(a, b, axis):
    """Largest relative error over the slices along `axis` (columns for axis=0)."""
    num = np.sqrt(np.nansum((a - b) ** 2, axis=axis))
    den = np.sqrt(np.nansum(b ** 2, axis=axis))
    return float(np.max(num[den > 0] / den[den > 0]))


T_, H_, E_, I_ = 64, 64, 3, 64


def test_mx_fc1_quantises_along_h():
    """fc1: x and W1 blocked along H. Both are exact along H (and span 2^30 across tokens /
    2I), so a and u equal the bf16 step's bit for bit."""
    rng = np.random.default_rng(7)
    x = _exact_along((T_, H_), 1, rng)
    dy = _exact_along((T_, H_), 1, rng)
    w1 = np.stack([_exact_along((2 * I_, H_), 1, rng) for _ in range(E_)])
    w2 = np.stack([_exact_along((H_, I_), 1, rng) for _ in range(E_)])
    idx, fm, fb, bm, bb = _step(x, dy, w1, w2, rng)
    np.testing.assert_array_equal(fm["a"], fb["a"])
    np.testing.assert_array_equal(fm["u"], fb["u"])
    assert not np.array_equal(mx.mx(w1[0], axis=0), w1[0])     # the wrong axis would flush


def test_mx_fc2_quantises_along_i():
    """fc2: h and W2 blocked along I. W2 is exact along I and spans 2^30 across H, so no
    column of the fc2 output may be flushed, which blocking W2 along H would do."""
    rng = np.random.default_rng(14)
    x = orc.bf16_round(rng.standard_normal((T_, H_)))
    dy = orc.bf16_round(rng.standard_normal((T_, H_)))
    w1 = np.stack([orc.bf16_round(rng.standard_normal((2 * I_, H_)) / 8) for _ in range(E_)])
    w2 = np.stack([_exact_along((H_, I_), 1, rng) for _ in range(E_)])
    idx, fm, fb, bm, bb = _step(x, dy, w1, w2, rng)
    assert _worst_rel(fm["p"], fb["p"], axis=0) < 0.25
    assert not np.array_equal(mx.mx(w2[0], axis=0), w2[0])


def test_mx_dgate_is_inner_product_of_quantised_dh_result():
    """dh: dY blocked along H, W2^T blocked along H. Both exact along H, so the d-gate equals
    the exact <dY_t W2[e], h_s> (the fused form); blocking W2 along I would flush columns."""
    rng = np.random.default_rng(8)
    x = _exact_along((T_, H_), 1, rng)
    dy = _exact_along((T_, H_), 1, rng)
    w1 = np.stack([_exact_along((2 * I_, H_), 1, rng) for _ in range(E_)])
    w2 = np.stack([_exact_along((H_, I_), 0, rng) for _ in range(E_)])
    idx, fm, fb, bm, bb = _step(x, dy, w1, w2, rng)
    flat = idx.ravel()
    for s in range(flat.size):
        exact = np.dot(dy[s // 2] @ w2[flat[s]], fm["h"][s])
        assert abs(bm["dgate"].ravel()[s] - exact) <= 1e-12 * max(1.0, abs(exact))
    assert not np.array_equal(mx.mx(w2[0], axis=1), w2[0])


def test_mx_dx_quantises_along_2i():
    """dx: dGU blocked along 2I, W1^T blocked along 2I. W1 exact along 2I and spanning 2^30
    across H: no column of the dX partials may be flushed."""
    rng = np.random.default_rng(11)
    x = orc.bf16_round(rng.standard_normal((T_, H_)))
    dy = orc.bf16_round(rng.standard_normal((T_, H_)))
    w1 = np.stack([_exact_along((2 * I_, H_), 0, rng) for _ in range(E_)])
    w2 = np.stack([orc.bf16_round(rng.standard_normal((H_, I_)) / 8) for _ in range(E_)])
    idx, fm, fb, bm, bb = _step(x, dy, w1, w2, rng)
    assert _worst_rel(bm["q"], bb["q"], axis=0) < 0.25


def test_mx_weight_gradients_quantise_along_tokens():
    """dw2: dO and h blocked along tokens; dw1: dGU and x blocked along tokens. dY and x
    span 2^30 across H (constant along tokens): no row of dW2 and no column of dW1 may be
    flushed, which blocking along H would do."""
    rng = np.random.default_rng(12)
    x = _exact_along((T_, H_), 0, rng)
    dy = _exact_along((T_, H_), 0, rng)
    w1 = np.stack([orc.bf16_round(rng.standard_normal((2 * I_, H_)) / 8) for _ in range(E_)])
    w2 = np.stack([orc.bf16_round(rng.standard_normal((H_, I_)) / 8) for _ in range(E_)])
    idx, fm, fb, bm, bb = _step(x, dy, w1, w2, rng)
    for e in range(E_):
        if np.any(idx == e):
            assert _worst_rel(bm["dw2"][e], bb["dw2"][e], axis=1) < 0.25
            assert _worst_rel(bm["dw1"][e], bb["dw1"][e], axis=0) < 0.25


@pytest.mark.filterwarnings("ignore:overflow encountered in exp")
def test_mx_step_is_row_local():
    """No per-tensor or cross-token scale in the data path: scaling one token's input and
    output gradient by 2^12 leaves every other token's y and dX bit-identical."""
    rng = np.random.default_rng(13)
    x = orc.bf16_round(rng.standard_normal((T_, H_)))
    dy = orc.bf16_round(rng.standard_normal((T_, H_)))
    w1 = np.stack([orc.bf16_round(rng.standard_normal((2 * I_, H_)) / 8) for _ in range(E_)])
    w2 = np.stack([orc.bf16_round(rng.standard_normal((H_, I_)) / 8) for _ in range(E_)])
    _, f0, _, b0, _ = _step(x, dy, w1, w2, np.random.default_rng(1))
    x2, dy2 = x.copy(), dy.copy()
    x2[5] *= 2.0**12
    dy2[5] *= 2.0**12
    _, f1, _, b1, _ = _step(x2, dy2, w1, w2, np.random.default_rng(1))
    keep = np.arange(T_) != 5
    np.testing.assert_array_equal(f1["y"][keep], f0["y"][keep])
    np.testing.assert_array_equal(b1["dx"][keep], b0["dx"][keep])


def test_mx_token_blocks_restart_at_segment_starts():
    """Rows of each segment are exact in 32-row blocks aligned to the segment start but
    span 2^40 between segments; misaligned blocking (a global offset) would flush them."""
    rng = np.random.default_rng(9)
    segs = [45, 7, 70]
    rows = []
    for n in segs:
        pad = -(-n // 32) * 32
        blk = rng.integers(-7, 8, (pad, 16)).astype(np.float64) / 8.0
        mags = np.exp2(rng.integers(-40, 1, pad // 32).astype(np.float64))
        rows.append((blk * np.repeat(mags, 32)[:, None])[:n])
    r = np.concatenate(rows)
    np.testing.assert_array_equal(mx.mx_token_blocks(r, segs), r)
    assert not np.array_equal(mx.mx_token_blocks(r, [sum(segs)]), r)


def test_mx_step_close_to_bf16_step_on_random_inputs():
    """On random bf16 inputs the MX step stays within the MXFP8 error level of the bf16 step
    (loose statistical check: rel. Frobenius < 0.1)."""
    rng = np.random.default_rng(10)
    T, H, E, k, I = 64, 128, 4, 2, 128
    x = orc.bf16_round(rng.standard_normal((T, H)))
    dy = orc.bf16_round(rng.standard_normal((T, H)))
    wr = orc.bf16_round(rng.standard_normal((E, H)) / np.sqrt(H))
    w1 = orc.bf16_round(rng.standard_normal((E, 2 * I, H)) / np.sqrt(H))
    w2 = orc.bf16_round(rng.standard_normal((E, H, I)) / np.sqrt(I))
    z, idx, g = orc.route(x, wr, k)
    W = orc.DenseWeights(w1, w2)
    fm, fb = mx.forward_mx(x, W, idx, g, E, I), orc.forward(x, W, idx, g, "bf16", E, I)
    bm, bb = mx.backward_mx(x, W, wr, idx, g, fm, dy, I), orc.backward(x, W, wr, idx, g, fb, dy, "bf16", I)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(fm["y"], fb["y"]) < 0.1
    assert rel(bm["dx"], bb["dx"]) < 0.1
    assert rel(bm["dw1"][0], bb["dw1"][0]) < 0.1


# ---------------------------------------------------------------------------------------
# Flush pins: one operand of one GEMM gets an element 2^24 larger than the rest of its
# 32-block (a shared E8M0 scale then sends the rest below half the smallest E4M3 or
# E2M1 subnormal, so they quantise to exact zeros; each pin runs for both formats); the other operand is zero where the large
# elements sit, so an output the rest alone would feed must be exactly 0. An operand that
# is not quantised, or quantised along another axis, leaves it non-zero.
# ---------------------------------------------------------------------------------------

BIG = 2.0**24
HUGE = 2.0**40                          # where a product of small factors must stay > BIG
TF, HF, EF, IF = 32, 64, 3, 64          # at most 32 rows per expert: one token block each
J_H = [0, 32]                           # one position per 32-block along H
J_I = [0, 32]                           # ... along I


def _base(seed):
    rng = np.random.default_rng(seed)
    x = orc.bf16_round(rng.standard_normal((TF, HF)))
    dy = orc.bf16_round(rng.standard_normal((TF, HF)))
    w1 = orc.bf16_round(rng.standard_normal((EF, 2 * IF, HF)) / 8)
    w2 = orc.bf16_round(rng.standard_normal((EF, HF, IF)) / 8)
    return rng, x, dy, w1, w2


def _run(rng, x, dy, w1, w2, fmt="e4m3"):
    with np.errstate(over="ignore"):
        return _step(x, dy, w1, w2, rng, E=EF, k=2, I=IF, fmt=fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_fc1_x_along_h(fmt):
    rng, x, dy, w1, w2 = _base(21)
    x[:, J_H] = BIG
    w1[:, :, J_H] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(fm["a"] == 0) and np.all(fm["u"] == 0)
    assert np.any(fb["a"] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_fc1_w1_along_h(fmt):
    rng, x, dy, w1, w2 = _base(22)
    w1[:, :, J_H] = BIG
    x[:, J_H] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(fm["a"] == 0) and np.all(fm["u"] == 0)
    assert np.any(fb["a"] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_fc2_h_along_i(fmt):
    rng, x, dy, w1, w2 = _base(23)
    x[:, 0] = 1.0
    for i in J_I:                        # a_i = u_i = 2^12 > 0 for every token: h_i ~ 2^24
        w1[:, i, :] = 0
        w1[:, IF + i, :] = 0
        w1[:, i, 0] = w1[:, IF + i, 0] = 2.0**12
    w2[:, :, J_I] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(fm["p"] == 0) and np.all(fm["y"] == 0)
    assert np.any(fb["p"] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_fc2_w2_along_i(fmt):
    rng, x, dy, w1, w2 = _base(24)
    w1[:, J_I, :] = 0                    # a_i = 0 -> h_i = 0 at the large positions of W2
    w2[:, :, J_I] = BIG
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(fm["p"] == 0)
    assert np.any(fb["p"] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_dh_dy_along_h(fmt):
    """The dh result feeds both halves of dGU; with it flushed to zero, dGU is zero."""
    rng, x, dy, w1, w2 = _base(25)
    dy[:, J_H] = BIG
    w2[:, J_H, :] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(bm["dgu"] == 0) and np.all(bm["dgate"] == 0)
    assert np.any(bb["dgu"] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_dh_w2t_along_h(fmt):
    rng, x, dy, w1, w2 = _base(26)
    w2[:, J_H, :] = BIG
    dy[:, J_H] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(bm["dgu"] == 0)
    assert np.any(bb["dgu"] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_dx_dgu_along_2i(fmt):
    """dA_i large at i in J_I (large W2 columns) makes dGU large at da_i and du_i, one per
    32-block along 2I; W1 rows at those positions are zero on the upper half of H."""
    rng, x, dy, w1, w2 = _base(27)
    w2[:, :, J_I] = HUGE
    x[:, 0] = 1.0
    J = J_I + [IF + i for i in J_I]
    for j in J:                          # a = u = 1 at the large positions
        w1[:, j, :] = 0
        w1[:, j, 0] = 1.0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(bm["q"][:, HF // 2:] == 0)
    assert np.any(bb["q"][:, HF // 2:] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_dx_w1t_along_2i(fmt):
    rng, x, dy, w1, w2 = _base(28)
    J = J_I + [IF + i for i in J_I]
    w1[:, J, :] = BIG
    w2[:, :, J_I] = 0                    # dA_i = 0 -> dGU = 0 at the large positions of W1
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    assert np.all(bm["q"] == 0)
    assert np.any(bb["q"] != 0)


def _experts_of(idx, t):
    return sorted(set(idx[t].tolist()))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_dw_x_and_h_along_tokens(fmt):
    """Token 3's x is 2^24 in every column and W1's first column dominates, so its a, u
    and h are large and positive everywhere; its dY is zero, so its dGU and dO are zero: in
    each of its experts (one token block) both weight gradients vanish."""
    rng, x, dy, w1, w2 = _base(29)
    x[3] = BIG
    w1[:, :, 0] = 8.0
    dy[3] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    for e in _experts_of(idx, 3):
        assert np.all(bm["dw1"][e] == 0) and np.all(bm["dw2"][e] == 0), e
        assert np.any(bb["dw1"][e] != 0) and np.any(bb["dw2"][e] != 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_flush_dw_dgu_and_do_along_tokens(fmt):
    """Token 3's dY is 2^40 larger (so are its dO and dGU, except du on the upper half of I,
    where its a is zero); its x is zero on the upper half of H and W1's gate rows of the
    upper half of I only see that half, so its h is zero there: in each of its experts dW2's
    upper-half columns and dW1's upper-half columns (rows other than that du) vanish."""
    rng, x, dy, w1, w2 = _base(30)
    dy[3] *= HUGE
    x[3, HF // 2:] = 0
    w1[:, IF // 2:IF, :HF // 2] = 0
    idx, fm, fb, bm, bb = _run(rng, x, dy, w1, w2, fmt)
    for e in _experts_of(idx, 3):
        # rows where token 3's dGU is non-zero and so dominates its token block (an E2M1
        # dot product can cancel to exactly 0: then the block keeps the other tokens)
        slot = [sl for sl in np.nonzero(idx.ravel() == e)[0] if sl // 2 == 3][0]
        rows = np.array([r for r in range(IF + IF // 2) if bm["dgu"][slot, r] != 0])
        assert len(rows) >= 0.9 * (IF + IF // 2), (e, len(rows))
        assert np.all(bm["dw1"][e][rows, HF // 2:] == 0), e
        assert np.all(bm["dw2"][e][:, IF // 2:] == 0), e
        assert np.any(bb["dw1"][e][rows, HF // 2:] != 0) and np.any(bb["dw2"][e][:, IF // 2:] != 0)


def test_mx_expert_subset_matches_full_step():
    """Restricting the MX step to some experts reproduces their slots of the full step."""
    rng, x, dy, w1, w2 = _base(31)
    wr = rng.standard_normal((EF, HF)) * 0.2
    z, idx, g = orc.route(x, wr, 2, exact=True)
    W = orc.DenseWeights(w1, w2)
    f = mx.forward_mx(x, W, idx, g, EF, IF)
    b = mx.backward_mx(x, W, wr, idx, g, f, dy, IF)
    fe = mx.forward_mx(x, W, idx, g, EF, IF, experts=[1])
    be = mx.backward_mx(x, W, wr, idx, g, fe, dy, IF, experts=[1])
    s = np.nonzero(idx.ravel() == 1)[0]
    for n in ("a", "u", "h", "p"):
        np.testing.assert_array_equal(fe[n][s], f[n][s])
    np.testing.assert_array_equal(be["dgate"].ravel()[s], b["dgate"].ravel()[s])
    np.testing.assert_array_equal(be["dw1"][1], b["dw1"][1])
    np.testing.assert_array_equal(be["dw2"][1], b["dw2"][1])


def test_mx_storage_points_hand_worked():
    """Hand-worked MXFP8 example of the storage points.

    Forward: x = [1, 2^-10, 0, ...] (H = 32), W1 gate row [1, 1, 0, ...], up row [2, 4, 0, ...]
    are exact under MX quantisation (block scales 2^-8 and 2^-6, elements 256, 0.25 and
    128, 256), so a = 1 + 2^-10 and u = 2 + 2^-8 as in the bf16 example and the stored
    h is 1.46875, not the 1.4609375 that rounded a and u would give.

    Backward: dO = g*dY is rounded to bf16 before its token-axis MX blocks. Tokens with
    gate 0.75 and dY = 0.95703125 and -1 give dO = 0.7177734375 = 367.5 * 2^-9 and -0.75.
    The block scale is 2^-9 (amax 0.75). The bf16 value is 368 * 2^-9, an E4M3 tie between
    352 and 384 that goes to the even 384, so with stored h = 1 for both tokens dW2 = 0;
    quantising the unrounded 367.5 would give 352 and dW2 = -32 * 2^-9 = -0.0625."""
    H, I = 32, 32
    x = np.zeros((1, H))
    x[0, :2] = [1.0, 2.0 ** -10]
    w1 = np.zeros((1, 2 * I, H))
    w1[0, 0, :2] = [1.0, 1.0]
    w1[0, I, :2] = [2.0, 4.0]
    W = orc.DenseWeights(w1, np.ones((1, H, I)))
    f = mx.forward_mx(x, W, np.zeros((1, 1), np.int32), np.ones((1, 1)), 1, I)
    assert f["a"][0, 0] == 1.0 and f["u"][0, 0] == 2.0 and f["h"][0, 0] == 1.46875

    T = 2
    xs = np.ones((T, H))
    dy = np.zeros((T, H))
    dy[:, 0] = [0.95703125, -1.0]
    fwd = dict(a=np.ones((T, I)), u=np.ones((T, I)), h=np.ones((T, I)))
    b = mx.backward_mx(xs, W, np.zeros((1, H)), np.zeros((T, 1), np.int32), np.full((T, 1), 0.75), fwd, dy, I,
                        router=False)
    assert np.all(b["dw2"][0][0] == 0.0)
