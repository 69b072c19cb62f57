"""Pins of the token-shift oracle (RWKV-LLM page, "Time-mixing block", eqs. (11)-(13): the
projection inputs interpolate linearly between the current and the previous token).

The forward is pinned by its two end points (mu = 1 keeps the current token, mu = 0 the
previous one), by being affine in mu, and by chaining through x_prev.  The backward is pinned
by the exact adjoint identity of a linear map, <g, F(v)> = <F^T g, v>, in x, x_prev and mu
separately, and by torch fp64 autograd of the interpolation.
"""

import numpy as np
import pytest

import oracle
from linear_recurrence_rnn_amd import workloads


def small(B=3, T=17, C=5, M=3, seed=7):
    return workloads.make_token_shift(B, T, C, M, seed, with_grad=True)


@pytest.mark.parametrize("with_prev", [False, True])
def test_end_points(with_prev):
    d = small()
    xp = d["x_prev"] if with_prev else None
    B, T, C = d["x"].shape
    ones = np.ones((2, C), np.float32)
    out1 = oracle.token_shift(d["x"], ones, xp)
    assert np.array_equal(out1[0], d["x"].astype(np.float64))
    out0 = oracle.token_shift(d["x"], 0 * ones, xp)
    prev = np.zeros((B, C)) if xp is None else xp.astype(np.float64)
    assert np.array_equal(out0[1][:, 0], prev)
    assert np.array_equal(out0[1][:, 1:], d["x"][:, :-1].astype(np.float64))


def test_affine_in_mu():
    d = small()
    C = d["x"].shape[2]
    ones = np.ones((1, C), np.float32)
    o0 = oracle.token_shift(d["x"], 0 * ones, d["x_prev"])[0]
    o1 = oracle.token_shift(d["x"], ones, d["x_prev"])[0]
    out = oracle.token_shift(d["x"], d["mu"], d["x_prev"])
    for m in range(d["mu"].shape[0]):
        mm = d["mu"][m].astype(np.float64)
        np.testing.assert_allclose(out[m], o0 + mm * (o1 - o0), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("split", [1, 8, 16])
def test_chains_through_x_prev(split):
    d = small()
    whole = oracle.token_shift(d["x"], d["mu"], d["x_prev"])
    a = oracle.token_shift(d["x"][:, :split], d["mu"], d["x_prev"])
    b = oracle.token_shift(d["x"][:, split:], d["mu"], d["x"][:, split - 1])
    assert np.array_equal(np.concatenate([a, b], axis=2), whole)


def _dot(a, b):
    return float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))


def test_adjoint_identity():
    """F is linear in (x, x_prev) and affine in mu: <g, dF> = <grad, d(input)> for every
    direction, exactly up to double rounding."""
    d = small(seed=11)
    rng = np.random.default_rng(12)
    g = d["g"]
    gx, gmu, gxp = oracle.token_shift_backward(d["x"], d["mu"], g, d["x_prev"])
    # x and x_prev: F(x, xp) is linear, so F(v, vp) is the directional derivative.
    v = rng.standard_normal(d["x"].shape).astype(np.float32)
    vp = rng.standard_normal(d["x_prev"].shape).astype(np.float32)
    lhs = _dot(g, oracle.token_shift(v, d["mu"], vp))
    assert abs(lhs - (_dot(gx, v) + _dot(gxp, vp))) <= 1e-10 * max(1.0, abs(lhs))
    # mu: F(mu + e_m,c delta) - F(mu) for a unit direction per entry (delta exact in float32).
    C = d["x"].shape[2]
    for m, c in ((0, 0), (1, C - 1), (2, 2)):
        mu2 = d["mu"].copy()
        mu2[m, c] = mu2[m, c] + np.float32(0.25)
        delta = float(mu2[m, c]) - float(d["mu"][m, c])
        diff = oracle.token_shift(d["x"], mu2, d["x_prev"]) - oracle.token_shift(d["x"], d["mu"], d["x_prev"])
        assert abs(_dot(g, diff) - gmu[m, c] * delta) <= 1e-10 * max(1.0, abs(gmu[m, c]))


def test_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    d = small(seed=13)
    gx, gmu, gxp = oracle.token_shift_backward(d["x"], d["mu"], d["g"], d["x_prev"])
    tx = torch.tensor(d["x"], dtype=torch.float64, requires_grad=True)
    tp = torch.tensor(d["x_prev"], dtype=torch.float64, requires_grad=True)
    tm = torch.tensor(d["mu"], dtype=torch.float64, requires_grad=True)
    shifted = torch.cat([tp[:, None, :], tx[:, :-1, :]], dim=1)
    out = torch.stack([torch.lerp(shifted, tx, tm[m]) for m in range(tm.shape[0])])
    (out * torch.tensor(d["g"], dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(gx, tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gmu, tm.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gxp, tp.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_empty_and_single_step():
    d = small(T=1)
    gx, gmu, gxp = oracle.token_shift_backward(d["x"], d["mu"], d["g"], d["x_prev"])
    mu = d["mu"].astype(np.float64)[:, None, None, :]
    np.testing.assert_allclose(gx[:, 0], np.sum(mu[:, :, 0] * d["g"][:, :, 0], axis=0), rtol=1e-14)
    np.testing.assert_allclose(gxp, np.sum((1 - mu[:, :, 0]) * d["g"][:, :, 0], axis=0), rtol=1e-14)
    e = small(T=0)
    assert oracle.token_shift(e["x"], e["mu"]).shape == (3, 3, 0, 5)
    gx, gmu, gxp = oracle.token_shift_backward(e["x"], e["mu"], e["g"], e["x_prev"])
    assert gx.shape == (3, 0, 5) and np.all(gmu == 0) and np.all(gxp == 0)

