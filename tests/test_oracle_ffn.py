"""Pins of the oracle's forward and backward against independent computations.

* E = 1, k = 1 reduces to a dense SwiGLU MLP (torch.nn.functional ops).
* Identical experts: the output does not depend on routing (gates sum to 1).
* Dense brute force: every expert evaluated for every token, masked by routing.
* torch.autograd in fp64 on that dense formulation: dX, dW1, dW2, dWr, d-gate.
* Central finite differences of L = <dY, y> on the smallest shapes.
Each test names the mistake it is there to catch.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as orc


def _problem(T=24, H=16, E=5, k=2, I=8, seed=0, same_experts=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) / np.sqrt(H)
    w1 = rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)
    w2 = rng.standard_normal((E, H, I)) / np.sqrt(I)
    if same_experts:
        w1[:] = w1[0]
        w2[:] = w2[0]
    bias = rng.standard_normal(E) * 0.3
    dy = rng.standard_normal((T, H))
    return x, wr, w1, w2, bias, dy


def _route_exact(x, wr, bias, k):
    z = orc.router_logits_exact(x, wr, bias)
    idx = orc.select_topk(z, k)
    return z, idx, orc.topk_gates(z, idx)


def _dense_torch(x, wr, w1, w2, bias, idx, I):
    """Dense masked formulation in torch fp64 (autograd-capable)."""
    z = x @ wr.T + bias
    g = torch.softmax(z.gather(1, idx), dim=1)
    outs = []
    for e in range(w1.shape[0]):
        a = x @ w1[e, :I].T
        u = x @ w1[e, I:].T
        outs.append((F.silu(a) * u) @ w2[e].T)
    allo = torch.stack(outs, 0)                        # [E, T, H]
    T = x.shape[0]
    y = torch.zeros_like(x)
    for j in range(idx.shape[1]):
        y = y + g[:, j:j + 1] * allo[idx[:, j], torch.arange(T)]
    return y, g


def test_single_expert_is_dense_swiglu():
    """E=1, k=1: catches swapped gate/up halves, a missing silu, or W2 applied transposed."""
    x, wr, w1, w2, bias, _ = _problem(E=1, k=1)
    I = 8
    z, idx, g = _route_exact(x, wr, bias, 1)
    assert np.all(g == 1.0)
    out = orc.forward(x, orc.DenseWeights(w1, w2), idx, g, "exact", 1, I)
    xt = torch.from_numpy(x)
    ref = F.linear(F.silu(F.linear(xt, torch.from_numpy(w1[0, :I]))) * F.linear(xt, torch.from_numpy(w1[0, I:])),
                   torch.from_numpy(w2[0]))
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_experts_output_independent_of_routing():
    """All experts equal: y = FFN(x). Catches gates that do not sum to one or a dropped slot."""
    I = 8
    x, wr, w1, w2, bias, _ = _problem(E=6, k=3, same_experts=True)
    z, idx, g = _route_exact(x, wr, bias, 3)
    out = orc.forward(x, orc.DenseWeights(w1, w2), idx, g, "exact", 6, I)
    a = x @ w1[0, :I].T
    u = x @ w1[0, I:].T
    ref = (orc.silu(a) * u) @ w2[0].T
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("E,k", [(5, 2), (8, 3), (4, 4)])
def test_forward_matches_dense_brute_force(E, k):
    """Every expert on every token, masked: catches a slot/expert mix-up or wrong gate index."""
    I = 8
    x, wr, w1, w2, bias, _ = _problem(E=E, k=k, seed=E + k)
    z, idx, g = _route_exact(x, wr, bias, k)
    out = orc.forward(x, orc.DenseWeights(w1, w2), idx, g, "exact", E, I)
    t = lambda a: torch.from_numpy(a)
    y, gt = _dense_torch(t(x), t(wr), t(w1), t(w2), t(bias), torch.from_numpy(idx.astype(np.int64)), I)
    np.testing.assert_allclose(g, gt.numpy(), rtol=1e-12)
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("E,k,seed", [(5, 2, 1), (8, 3, 2), (6, 1, 3), (4, 4, 4)])
def test_backward_matches_autograd_dense(E, k, seed):
    """torch.autograd on the dense formulation: catches a sign or index error in any
    gradient (dX incl. router term, dW1 halves, dW2, dWr, d-gate)."""
    I = 8
    x, wr, w1, w2, bias, dy = _problem(E=E, k=k, seed=seed)
    z, idx, g = _route_exact(x, wr, bias, k)
    W = orc.DenseWeights(w1, w2)
    fwd = orc.forward(x, W, idx, g, "exact", E, I)
    bwd = orc.backward(x, W, wr, idx, g, fwd, dy, "exact", I)
    t = lambda a: torch.from_numpy(a.copy()).requires_grad_(True)
    xt, wrt, w1t, w2t = t(x), t(wr), t(w1), t(w2)
    y, gt = _dense_torch(xt, wrt, w1t, w2t, torch.from_numpy(bias), torch.from_numpy(idx.astype(np.int64)), I)
    gt.retain_grad()
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(bwd["dgate"], gt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bwd["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bwd["dwr"], wrt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for e in range(E):
        np.testing.assert_allclose(bwd["dw1"][e], w1t.grad[e].numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(bwd["dw2"][e], w2t.grad[e].numpy(), rtol=1e-10, atol=1e-12)


def _loss(x, wr, w1, w2, bias, dy, idx, I):
    z = orc.router_logits_exact(x, wr, bias)
    g = orc.topk_gates(z, idx)
    out = orc.forward(x, orc.DenseWeights(w1, w2), idx, g, "exact", w1.shape[0], I)
    return float(np.sum(out["y"] * dy))


def test_backward_matches_finite_differences():
    """Central differences in fp64 (step 1e-6) on the tiny shapes, routing held fixed
    (tokens whose k-th/(k+1)-th logit gap is under 1e-3 are not perturbed)."""
    I, E, k = 8, 8, 2
    x, wr, w1, w2, bias, dy = _problem(T=16, H=12, E=E, k=k, I=I, seed=11)
    z, idx, g = _route_exact(x, wr, bias, k)
    zs = np.sort(z, axis=1)[:, ::-1]
    safe = (zs[:, k - 1] - zs[:, k]) > 1e-3
    W = orc.DenseWeights(w1, w2)
    fwd = orc.forward(x, W, idx, g, "exact", E, I)
    bwd = orc.backward(x, W, wr, idx, g, fwd, dy, "exact", I)
    rng = np.random.default_rng(0)
    eps = 1e-6

    def fd(arr_name, pos):
        arrs = dict(x=x, wr=wr, w1=w1, w2=w2)
        p = {n: a.copy() for n, a in arrs.items()}
        p[arr_name][pos] += eps
        lp = _loss(p["x"], p["wr"], p["w1"], p["w2"], bias, dy, idx, I)
        p[arr_name][pos] -= 2 * eps
        lm = _loss(p["x"], p["wr"], p["w1"], p["w2"], bias, dy, idx, I)
        return (lp - lm) / (2 * eps)

    checked = 0
    for _ in range(12):
        t = int(rng.integers(16))
        if not safe[t]:
            continue
        h = int(rng.integers(12))
        assert abs(fd("x", (t, h)) - bwd["dx"][t, h]) < 1e-6 * max(1, abs(bwd["dx"][t, h]))
        checked += 1
    assert checked >= 4
    # router rows: perturbing wr moves logits of every token; all must be safe
    if np.all(safe):
        for _ in range(6):
            e, h = int(rng.integers(E)), int(rng.integers(12))
            assert abs(fd("wr", (e, h)) - bwd["dwr"][e, h]) < 1e-6 * max(1, abs(bwd["dwr"][e, h]))
    for _ in range(8):
        e, r, h = int(rng.integers(E)), int(rng.integers(2 * I)), int(rng.integers(12))
        assert abs(fd("w1", (e, r, h)) - bwd["dw1"][e][r, h]) < 1e-6 * max(1, abs(bwd["dw1"][e][r, h]))
        e, h, i = int(rng.integers(E)), int(rng.integers(12)), int(rng.integers(I))
        assert abs(fd("w2", (e, h, i)) - bwd["dw2"][e][h, i]) < 1e-6 * max(1, abs(bwd["dw2"][e][h, i]))


def test_dgate_identity_fused_form():
    """The fused SwiGLU-backward form <dY W2, h> equals <dY, o> (to rounding in fp64)."""
    I, E, k = 8, 5, 2
    x, wr, w1, w2, bias, dy = _problem(E=E, k=k, seed=21)
    z, idx, g = _route_exact(x, wr, bias, k)
    W = orc.DenseWeights(w1, w2)
    fwd = orc.forward(x, W, idx, g, "exact", E, I)
    bwd = orc.backward(x, W, wr, idx, g, fwd, dy, "exact", I)
    flat = idx.ravel()
    for s in range(flat.size):
        t, e = s // k, flat[s]
        fused = np.dot(dy[t] @ w2[e], fwd["h"][s])
        assert abs(fused - bwd["dgate"].ravel()[s]) <= 1e-12 * max(1.0, abs(fused))


def test_storage_rounding_points_bf16():
    """bf16 storage: saved a/u/h, partials and outputs are bf16 values; y is the
    rounded slot-order sum of the rounded partials."""
    I, E, k = 8, 5, 2
    x, wr, w1, w2, bias, dy = _problem(E=E, k=k, seed=31)
    x = orc.bf16_round(x)
    z, idx, g = _route_exact(x, wr, bias, k)
    W = orc.DenseWeights(orc.bf16_round(w1), orc.bf16_round(w2))
    fwd = orc.forward(x, W, idx, g, "bf16", E, I)
    for name in ("a", "u", "h", "p", "y"):
        np.testing.assert_array_equal(fwd[name], orc.bf16_round(fwd[name]))
    y = np.zeros_like(x)
    for j in range(k):
        y += g[:, j:j + 1] * fwd["p"][j::k]
    np.testing.assert_array_equal(fwd["y"], orc.bf16_round(y))
    # h is rounded from the unrounded a, u (not from the stored ones)
    a = x[np.arange(x.shape[0]).repeat(k)]
    bwd = orc.backward(x, W, wr, idx, g, fwd, orc.bf16_round(dy), "bf16", I)
    for name in ("dgu", "q", "dx", "dwr"):
        v = bwd[name] if name != "dwr" else bwd[name]
        np.testing.assert_array_equal(v, orc.bf16_round(v))


def test_storage_points_hand_worked_h_from_unrounded_a_u():
    """Hand-worked example of where bf16 rounding happens in the forward: h is formed from
    the fp32 accumulators a and u, and only the stored a, u, h are rounded.

    x = [1, 2^-10], W1 gate row [1, 1], up row [2, 4]: a = 1 + 2^-10, u = 2 + 2^-8 exactly.
    Stored a, u round to 1 and 2 (both less than half a bf16 step away).
    h = silu(1 + 2^-10) * (2 + 2^-8) = 1.466788...; in steps of 2^-7 that is 187.749, so
    the stored h is 188 * 2^-7 = 1.46875 (silu(1) * 2 = 1.462117 = 187.151 steps would
    give 1.4609375: the mistake of forming h from the rounded a and u)."""
    x = np.array([[1.0, 2.0 ** -10]])
    w1 = np.array([[[1.0, 1.0], [2.0, 4.0]]])           # [E=1, 2I=2, H=2]
    w2 = np.array([[[1.0], [1.0]]])                      # [E=1, H=2, I=1]
    W = orc.DenseWeights(w1, w2)
    idx = np.zeros((1, 1), dtype=np.int32)
    fwd = orc.forward(x, W, idx, np.ones((1, 1)), "bf16", 1, 1)
    assert fwd["a"][0, 0] == 1.0 and fwd["u"][0, 0] == 2.0
    assert fwd["h"][0, 0] == 1.46875
    # o = W2 h from the stored h: both partial columns equal the stored h
    np.testing.assert_array_equal(fwd["p"][0], [1.46875, 1.46875])


def test_storage_points_hand_worked_do_rounded_before_dw2():
    """Hand-worked example: the dW2 operand dO = g*dY is stored (rounded to bf16) before the
    weight-gradient GEMM.

    Two tokens routed to the one expert with gate 0.625, H = I = 1, stored h = 1 for both,
    dY = 1.0234375 and -1. dO = 0.6396484375 (163.75 steps of 2^-8, so 164 * 2^-8 =
    0.640625 stored) and -0.625 (exact). dW2 = 0.640625 - 0.625 = 2^-6 exactly; with dO
    left unrounded it would be 0.0146484375 = 15 * 2^-10 (also a bf16 value, so the final
    rounding of dW2 keeps the two apart)."""
    T, I = 2, 1
    x = np.array([[1.0], [1.0]])
    W = orc.DenseWeights(np.ones((1, 2, 1)), np.ones((1, 1, 1)))
    idx = np.zeros((T, 1), dtype=np.int32)
    g = np.full((T, 1), 0.625)
    fwd = dict(a=np.ones((T, I)), u=np.ones((T, I)), h=np.ones((T, I)), o=np.ones((T, 1)))
    dy = np.array([[1.0234375], [-1.0]])
    b = orc.backward(x, W, np.zeros((1, 1)), idx, g, fwd, dy, "bf16", I, router=False)
    assert b["dw2"][0][0, 0] == 2.0 ** -6


@pytest.mark.parametrize("mx", [False, "e4m3", "e2m1"])
def test_expert_chunked_step_equals_whole_step(mx):
    """The threaded, expert-chunked evaluation the full-size GPU tests use (harness.
    oracle_step_parallel) gives the oracle's whole-step outputs bit for bit, here with an
    expert that has no slots and chunks of unequal size."""
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from harness import oracle_step_parallel
    T, H, E, k, I = 40, 32, 7, 3, 32
    x, wr, w1, w2, bias, dy = _problem(T=T, H=H, E=E, k=k, I=I, seed=5)
    bias[6] = -50.0                                  # expert 6 gets no slots
    x, dy = orc.bf16_round(x), orc.bf16_round(dy)
    z, idx, g = _route_exact(x, wr, bias, k)
    W = orc.DenseWeights(orc.bf16_round(w1), orc.bf16_round(w2))
    if mx:
        f0 = orc.mx.forward_mx(x, W, idx, g, E, I, fmt=mx)
        b0 = orc.mx.backward_mx(x, W, wr, idx, g, f0, dy, I, fmt=mx)
    else:
        f0 = orc.forward(x, W, idx, g, "bf16", E, I)
        b0 = orc.backward(x, W, wr, idx, g, f0, dy, "bf16", I)
    f1, b1 = oracle_step_parallel(x, W, wr, idx, g, dy, E, I, mx=mx, workers=3)
    for key in ("a", "u", "h", "p", "y"):
        np.testing.assert_array_equal(f1[key], f0[key], err_msg=key)
    for key in ("dgate", "dgu", "q", "dx", "dwr", "dz"):
        np.testing.assert_array_equal(b1[key], b0[key], err_msg=key)
    for e in range(E):
        if e in b1["dw1"]:
            np.testing.assert_array_equal(b1["dw1"][e], b0["dw1"][e])
            np.testing.assert_array_equal(b1["dw2"][e], b0["dw2"][e])
