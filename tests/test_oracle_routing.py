"""Pins of the oracle's routing and schedule against things other than itself.

Each test names the mistake it is there to catch.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc


def _round_fraction_f32(fr: Fraction) -> float:
    """Exact rational -> nearest float32 (ties to even), by integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** max(e - 23, -149)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(sign * fl * q)


def _brute_logit(xrow, wrow, b):
    acc = 0.0
    for xv, wv in zip(xrow, wrow):
        acc = _round_fraction_f32(Fraction(float(xv)) * Fraction(float(wv)) + Fraction(acc))
    if b is not None:
        acc = _round_fraction_f32(Fraction(acc) + Fraction(float(b)))
    return acc


def test_bf16_round_hand_values():
    """Catches a wrong significand width or a tie rule other than ties-to-even."""
    v = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3.0, 1 + 2**-7, 2**-133 * 2.5, 2**-133 * 3.5,
                  2**-134, 0.0, -0.0])
    want = np.array([1.0, 1.0, 1 + 2**-6, -1.0, 3.0, 1 + 2**-7, 2**-132, 2**-131, 0.0, 0.0, -0.0])
    np.testing.assert_array_equal(orc.bf16_round(v), want)


def test_bf16_round_matches_torch_on_float32_values():
    """Library routine: torch's float32 -> bfloat16 conversion rounds to nearest even."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(orc.bf16_round(v.astype(np.float64)), ref)


def test_router_logits_brute_force_fma_chain():
    """Exact rational fma chain on tiny inputs: catches a non-fused multiply-add,
    a different accumulation order, or the bias added at the wrong point."""
    rng = np.random.default_rng(1)
    T, H, E = 3, 37, 5
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    wr = torch.from_numpy((rng.standard_normal((E, H)) * 0.2).astype(np.float32)).to(torch.bfloat16).float().numpy()
    bias = (rng.standard_normal(E) * 0.7).astype(np.float32)
    for b in (None, bias):
        z = orc.router_logits(x, wr, b)
        for t in range(T):
            for e in range(E):
                assert z[t, e] == np.float32(_brute_logit(x[t], wr[e], None if b is None else b[e]))


def _brute_topk(zrow, k):
    """Textbook selection by repeated maximum with the stated total order."""
    def better(a, ea, b, eb):
        if np.isnan(b) and not np.isnan(a):
            return True
        if np.isnan(a):
            return np.isnan(b) and ea < eb
        return a > b or (a == b and ea < eb)

    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(zrow):
            if e in chosen:
                continue
            if best is None or better(v, e, zrow[best], best):
                best = e
        chosen.append(best)
    return chosen


def test_select_topk_brute_force_with_ties_zero_signs_nan():
    """Catches ties broken toward the higher index, -0/+0 treated as unequal, NaN ranked high."""
    rng = np.random.default_rng(2)
    E, k = 9, 4
    rows = []
    for _ in range(300):
        z = rng.integers(-3, 3, E).astype(np.float32)        # many exact ties
        if rng.random() < 0.3:
            z[rng.integers(E)] = np.nan
        if rng.random() < 0.3:
            z[rng.integers(E)] = -0.0
            z[rng.integers(E)] = 0.0
        rows.append(z)
    z = np.stack(rows)
    idx = orc.select_topk(z, k)
    for t in range(z.shape[0]):
        assert list(idx[t]) == _brute_topk(list(z[t]), k)


def test_zero_token_row_closed_form():
    """x_t = 0 makes every logit +0: experts 0..k-1 in order, gates exactly 1/k."""
    T, H, E, k = 4, 64, 16, 8
    rng = np.random.default_rng(3)
    x = np.zeros((T, H), np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    z, idx, g = orc.route(x, wr, k)
    assert np.all(z == 0)
    np.testing.assert_array_equal(idx, np.tile(np.arange(k), (T, 1)))
    np.testing.assert_array_equal(g, np.full((T, k), 1.0 / k))


def test_duplicate_router_rows_lower_index_wins():
    """Duplicated router rows produce exactly equal logits; the lower expert index must come first."""
    rng = np.random.default_rng(4)
    T, H, E, k = 50, 32, 6, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    wr[4] = wr[1]
    z, idx, g = orc.route(x, wr, k)
    assert np.all(z[:, 4] == z[:, 1])
    for t in range(T):
        if 1 in idx[t] or 4 in idx[t]:
            order = list(idx[t])
            assert 1 in order and (4 not in order or order.index(1) < order.index(4))
            if 4 in order:
                assert g[t, order.index(1)] == g[t, order.index(4)]


def test_gates_invariants():
    """Gates sum to 1 (within k ulp), are positive and non-increasing in slot order."""
    rng = np.random.default_rng(6)
    z = rng.standard_normal((500, 40)).astype(np.float32) * 3
    idx = orc.select_topk(z, 8)
    g = orc.topk_gates(z, idx)
    assert np.all(np.abs(g.sum(1) - 1) <= 8 * np.finfo(np.float64).eps)
    assert np.all(g > 0) and np.all(np.diff(g, axis=1) <= 0)
    # equals the full softmax renormalised over the selected experts
    full = np.exp(z.astype(np.float64) - z.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), 1)
    np.testing.assert_allclose(g, sel / sel.sum(1, keepdims=True), rtol=1e-12)


@pytest.mark.parametrize("E,k,BM", [(8, 2, 32), (32, 2, 64), (50, 8, 128), (5, 5, 4)])
def test_schedule_against_stable_argsort(E, k, BM):
    """Library routine: numpy's stable argsort of the flat expert ids is the permutation.
    Also: bijection, counts sum to T*k, exclusive offsets, tiles cover each row once."""
    rng = np.random.default_rng(E * 100 + k)
    T = 97
    z = rng.standard_normal((T, E)).astype(np.float32)
    z[:, 0] += 2.0                                   # one hot expert
    if E > 3:
        z[:, 3] = -50                                # a never-chosen expert when k < E
    idx = orc.select_topk(z, k)
    sc = orc.schedule(idx, E, BM)
    flat = idx.ravel()
    np.testing.assert_array_equal(sc["perm"], np.argsort(flat, kind="stable"))
    assert sorted(sc["perm"].tolist()) == list(range(T * k))
    np.testing.assert_array_equal(sc["inv"][sc["perm"]], np.arange(T * k))
    assert sc["counts"].sum() == T * k
    np.testing.assert_array_equal(sc["counts"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(sc["offsets"], np.concatenate([[0], np.cumsum(sc["counts"])]))
    cover = np.zeros(T * k, int)
    for e, r0, n in sc["tiles"]:
        assert 1 <= n <= BM
        assert sc["offsets"][e] <= r0 and r0 + n <= sc["offsets"][e + 1]
        cover[r0:r0 + n] += 1
    assert np.all(cover == 1)
    assert len(sc["tiles"]) == sum(-(-c // BM) for c in sc["counts"])
    # tokens ascend within each expert (stable)
    for e in range(E):
        seg = sc["perm"][sc["offsets"][e]:sc["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
