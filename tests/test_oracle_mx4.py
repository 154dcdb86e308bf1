"""Pins of the oracle's MXFP4 quantisation (OCP MX v1.0 FP4 E2M1 elements under the
E8M0 scale of 32-element blocks). The quantisation points of the layer step are
MXFP8's; the flush pins of test_oracle_mx.py run for both element formats."""
import numpy as np

import oracle as orc
from oracle import mx

# E2M1 magnitudes by code (sign bit apart): exponent bits 2..1 (bias 1), mantissa bit 0
E2M1_BY_CODE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute_e2m1(v):
    """Nearest E2M1 value by exhaustive search over the eight magnitudes; a tie goes to
    the magnitude whose code has mantissa bit 0; beyond 6 saturates."""
    out = np.empty_like(v)
    for i, x in enumerate(v):
        a = abs(x)
        if a >= 6.0:
            m = 6.0
        else:
            d = [abs(a - g) for g in E2M1_BY_CODE]
            best = min(d)
            cands = [c for c in range(8) if d[c] == best]
            m = E2M1_BY_CODE[[c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]]
        out[i] = -m if x < 0 else m
    return out


def test_e2m1_rounding_brute_force():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    v = np.array(mids + [-m for m in mids] + E2M1_BY_CODE + [7.0, 7.9, 100.0, -6.5, 0.2, 0.3, 5.1, 4.9])
    rng = np.random.default_rng(0)
    v = np.concatenate([v, rng.uniform(-8, 8, 20000), rng.uniform(-1, 1, 5000)])
    np.testing.assert_array_equal(mx.e2m1_round(v), _brute_e2m1(v))
    # the hand values of the ties: to the even mantissa
    np.testing.assert_array_equal(mx.e2m1_round(np.array(mids)), [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])


def test_mx4_scale_rule_hand_examples():
    """s = floor(log2 amax) - 2: amax 1.0 -> s = -2 (elements are 4 v), saturation at 6,
    subnormal ties, zero block, a block far below 1."""
    blk = np.zeros(32)
    blk[:7] = [1.0, 0.9, 0.3, 0.1, 0.0625, 0.1875, -0.8]
    el, s = mx.mx_quantize(blk, fmt="e2m1")
    assert s.tolist() == [-2]
    # 4, 3.6 -> 4 (step 1 in [2, 4)), 1.2 -> 1 (step 0.5), 0.4 -> 0.5, 0.25 -> 0 (tie to
    # even), 0.75 -> 1 (tie to even), -3.2 -> -3
    assert el[:7].tolist() == [4.0, 4.0, 1.0, 0.5, 0.0, 1.0, -3.0]
    blk[0] = 1.9                                  # 7.6 > 6: saturates
    el, s = mx.mx_quantize(blk, fmt="e2m1")
    assert s.tolist() == [-2] and el[0] == 6.0
    el, s = mx.mx_quantize(np.zeros(64), fmt="e2m1")
    assert s.tolist() == [-127, -127] and np.all(el == 0)
    el, s = mx.mx_quantize(np.full(32, -3.0 * 2.0**-100), fmt="e2m1")
    assert s.tolist() == [-101] and np.all(el == -6.0)
    # the same block under E4M3 keeps a different scale: the format's emax is what differs
    assert mx.mx_quantize(np.full(32, 1.0))[1].tolist() == [-8]
    assert mx.mx_quantize(np.full(32, 1.0), fmt="e2m1")[1].tolist() == [-2]


def test_mx4_idempotent_and_error_bound():
    """Quantising a quantised tensor changes nothing; unsaturated elements are within half
    a step: relative 2^-2 for normals, absolute 2^(s-2) for subnormals."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((40, 256)) * np.exp2(rng.uniform(-8, 8, (40, 1)))
    q = mx.mx(v, fmt="e2m1")
    np.testing.assert_array_equal(mx.mx(q, fmt="e2m1"), q)
    el, s = mx.mx_quantize(v, fmt="e2m1")
    sc = np.repeat(np.exp2(s.astype(float)), 32, axis=1)
    ok = np.abs(v / sc) <= 6
    err = np.abs(q - v)
    assert np.all(err[ok] <= np.maximum(np.abs(v[ok]) * 2.0**-2, sc[ok] * 2.0**-2) * (1 + 1e-12))
    assert np.all(np.isin(np.abs(el), E2M1_BY_CODE))


def _exact4_along_h(rows, H, rng, spread=30):
    """Rows exactly representable in E2M1 blocks along H: E2M1 values times 2^m, m fixed
    per row and spanning 2^spread over the rows, every block holding a +-4 or +-6 (so its
    scale is 2^m)."""
    v = rng.choice(np.array(E2M1_BY_CODE[:7]), size=(rows, H)) * rng.choice([-1.0, 1.0], size=(rows, H))
    v[:, ::32] = rng.choice([-6.0, -4.0, 4.0, 6.0], size=(rows, H // 32))
    m = np.exp2(rng.integers(-spread, 1, rows).astype(np.float64))
    return v * m[:, None]


def test_mx4_fc1_quantises_along_h_exactly():
    """fc1 with x and W1 exact along H under E2M1: a and u equal the bf16 step's bit for
    bit; the same W1 blocked along the other axis would not be exact."""
    rng = np.random.default_rng(7)
    T, H, E, I, k = 48, 64, 3, 64, 2
    x = _exact4_along_h(T, H, rng)
    w1 = np.stack([_exact4_along_h(2 * I, H, rng) for _ in range(E)])
    w2 = orc.bf16_round(rng.standard_normal((E, H, I)) / 8)
    wr = rng.standard_normal((E, H)) * 0.2
    z, idx, g = orc.route(x, wr, k, exact=True)
    W = orc.DenseWeights(w1, w2)
    with np.errstate(over="ignore"):
        f4 = mx.forward_mx(x, W, idx, g, E, I, fmt="e2m1")
        fb = orc.forward(x, W, idx, g, "bf16", E, I)
    np.testing.assert_array_equal(f4["a"], fb["a"])
    np.testing.assert_array_equal(f4["u"], fb["u"])
    assert not np.array_equal(mx.mx(w1[0], axis=0, fmt="e2m1"), w1[0])


def test_mx4_step_follows_bf16_step_loosely():
    """On random inputs the MXFP4 step stays within the coarse error of a 1-bit mantissa
    (each operand relative error up to 1/4) of the bf16 step, and further than MXFP8."""
    rng = np.random.default_rng(3)
    T, H, E, k, I = 64, 64, 4, 2, 64
    x = orc.bf16_round(rng.standard_normal((T, H)))
    dy = orc.bf16_round(rng.standard_normal((T, H)))
    wr = orc.bf16_round(rng.standard_normal((E, H)) / np.sqrt(H))
    w1 = orc.bf16_round(rng.standard_normal((E, 2 * I, H)) / np.sqrt(H))
    w2 = orc.bf16_round(rng.standard_normal((E, H, I)) / np.sqrt(I))
    z, idx, g = orc.route(x, wr, k)
    W = orc.DenseWeights(w1, w2)
    fb = orc.forward(x, W, idx, g, "bf16", E, I)
    bb = orc.backward(x, W, wr, idx, g, fb, dy, "bf16", I)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    errs = {}
    for fmt in ("e4m3", "e2m1"):
        f = mx.forward_mx(x, W, idx, g, E, I, fmt=fmt)
        b = mx.backward_mx(x, W, wr, idx, g, f, dy, I, fmt=fmt)
        errs[fmt] = (rel(f["y"], fb["y"]), rel(b["dx"], bb["dx"]), rel(b["dw1"][0], bb["dw1"][0]))
    assert all(e < 0.5 for e in errs["e2m1"]), errs
    assert all(e4 < e2 for e4, e2 in zip(errs["e4m3"], errs["e2m1"])), errs
