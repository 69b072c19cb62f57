"""Pins of the oracle's scan backward (adjoints of x_t = a_t x_{t-1} + b_t and of
x_t = lam x_{t-1} + u_t; the pages give no backward, the adjoint is derived from the scan
forms on the minGRU page and in the LRU write-up, eq. lr-xx).

Each pin is independent of the oracle's C code: torch autograd on a plain loop, the
unrolled O(T^2) sums, central finite differences of a Python forward, and special cases
with closed forms (a = 1: reverse cumulative sum; a = 0: no carry; theta = 0: the real
scan's adjoint).
"""

import math

import numpy as np
import pytest

import brute
import oracle
from linear_recurrence_rnn_amd import workloads

torch = pytest.importorskip("torch")


def _real_case(seed, B=2, T=13, C=3, with_x0=True, a_range=(-1.2, 1.2)):
    rng = np.random.default_rng(seed)
    a = rng.uniform(*a_range, (B, T, C)).astype(np.float32)
    b = rng.standard_normal((B, T, C)).astype(np.float32)
    g = rng.standard_normal((B, T, C)).astype(np.float32)
    x0 = rng.standard_normal((B, C)).astype(np.float32) if with_x0 else None
    return a, b, g, x0


def _cplx_case(seed, B=2, T=11, C=3, with_x0=True):
    rng = np.random.default_rng(seed)
    d = workloads.make_lru(B, T, C, seed, 0.5, 1.0, 2 * math.pi)
    g = (rng.standard_normal((B, T, C)) + 1j * rng.standard_normal((B, T, C))).astype(np.complex64)
    x0 = ((rng.standard_normal((B, C)) + 1j * rng.standard_normal((B, C))).astype(np.complex64)
          if with_x0 else None)
    return d["lam"], d["u"], g, x0


@pytest.mark.parametrize("with_x0", [True, False])
def test_real_backward_matches_autograd(with_x0):
    a, b, g, x0 = _real_case(1, with_x0=with_x0)
    x = oracle.scan_real(a, b, x0)
    ga, gb, gx0 = oracle.scan_real_backward(a, x, g, x0)
    ta = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tb = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    tx0 = None if x0 is None else torch.tensor(x0, dtype=torch.float64, requires_grad=True)
    brute.scan_torch(ta, tb, tx0).backward(torch.tensor(g, dtype=torch.float64))
    np.testing.assert_allclose(ga, ta.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gb, tb.grad.numpy(), rtol=1e-12, atol=1e-13)
    if x0 is None:
        assert gx0 is None
    else:
        np.testing.assert_allclose(gx0, tx0.grad.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("with_x0", [True, False])
def test_complex_backward_matches_autograd(with_x0):
    lam, u, g, x0 = _cplx_case(2, with_x0=with_x0)
    x = oracle.scan_complex(lam, u, x0)
    glam, gu, gx0 = oracle.scan_complex_backward(lam, x, g, x0)
    tl = torch.tensor(lam, dtype=torch.complex128, requires_grad=True)
    tu = torch.tensor(u, dtype=torch.complex128, requires_grad=True)
    tx0 = None if x0 is None else torch.tensor(x0, dtype=torch.complex128, requires_grad=True)
    brute.scan_torch(tl, tu, tx0).backward(torch.tensor(g, dtype=torch.complex128))
    np.testing.assert_allclose(glam, tl.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gu, tu.grad.numpy(), rtol=1e-12, atol=1e-13)
    if x0 is not None:
        np.testing.assert_allclose(gx0, tx0.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_real_backward_unrolled_sums():
    a, b, g, x0 = _real_case(3, T=17)
    x = oracle.scan_real(a, b, x0)
    for mine, ref in zip(oracle.scan_real_backward(a, x, g, x0), brute.scan_real_backward_sums(a, g, x, x0)):
        np.testing.assert_allclose(mine, ref, rtol=1e-11, atol=1e-12)


def test_complex_backward_unrolled_sums():
    lam, u, g, x0 = _cplx_case(4, T=15)
    x = oracle.scan_complex(lam, u, x0)
    for mine, ref in zip(oracle.scan_complex_backward(lam, x, g, x0),
                         brute.scan_complex_backward_sums(lam, g, x, x0)):
        np.testing.assert_allclose(mine, ref, rtol=1e-11, atol=1e-12)


def test_real_backward_finite_differences():
    # L = sum g x; perturb single entries of a, b, x0 in a float64 Python forward.
    a, b, g, x0 = _real_case(5, B=1, T=9, C=2)
    ad, bd, gd, x0d = (np.asarray(z, np.float64) for z in (a, b, g, x0))

    def loss(a_, b_, x0_):
        s, tot = x0_.copy(), 0.0
        for t in range(a_.shape[1]):
            s = a_[:, t] * s + b_[:, t]
            tot += float((gd[:, t] * s).sum())
        return tot

    x = oracle.scan_real(a, b, x0)
    ga, gb, gx0 = oracle.scan_real_backward(a, x, g, x0)
    h = 1e-6
    for (t, c) in [(0, 0), (4, 1), (8, 0)]:
        for arr, grad in ((ad, ga), (bd, gb)):
            p, m = arr.copy(), arr.copy()
            p[0, t, c] += h
            m[0, t, c] -= h
            args_p = (p, bd, x0d) if arr is ad else (ad, p, x0d)
            args_m = (m, bd, x0d) if arr is ad else (ad, m, x0d)
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[0, t, c]) < 1e-7 * max(1.0, abs(fd))
    p, m = x0d.copy(), x0d.copy()
    p[0, 1] += h
    m[0, 1] -= h
    fd = (loss(ad, bd, p) - loss(ad, bd, m)) / (2 * h)
    assert abs(fd - gx0[0, 1]) < 1e-7 * max(1.0, abs(fd))


def test_real_backward_special_cases():
    a, b, g, _ = _real_case(6, T=10)
    ones = np.ones_like(a)
    x = oracle.scan_real(ones, b)
    _, gb, _ = oracle.scan_real_backward(ones, x, g)
    # a = 1: gb is the reverse cumulative sum of g.
    np.testing.assert_allclose(gb, np.cumsum(g[:, ::-1].astype(np.float64), axis=1)[:, ::-1], rtol=1e-13, atol=1e-13)
    zeros = np.zeros_like(a)
    x = oracle.scan_real(zeros, b)
    ga, gb, _ = oracle.scan_real_backward(zeros, x, g)
    # a = 0: no carry between steps, gb = g, ga_t = g_t x_{t-1} = g_t b_{t-1}.
    np.testing.assert_array_equal(gb, g.astype(np.float64))
    np.testing.assert_allclose(ga[:, 1:], g[:, 1:].astype(np.float64) * b[:, :-1], rtol=1e-15)
    np.testing.assert_array_equal(ga[:, 0], 0.0)


def test_complex_backward_zero_phase_is_real_backward():
    # lam real (theta = 0) and real inputs: the complex adjoint is the real one with
    # a = lam, and glam is the sum of ga over batch and time.
    a, b, g, x0 = _real_case(7, a_range=(0.5, 0.99))
    lam = a[0, 0].astype(np.complex64)
    a_full = np.broadcast_to(a[0, 0], a.shape).astype(np.float32)
    x = oracle.scan_real(a_full, b, x0)
    ga, gb, gx0 = oracle.scan_real_backward(a_full, x, g, x0)
    xc = oracle.scan_complex(lam, b.astype(np.complex64), x0.astype(np.complex64))
    glam, gu, gxc0 = oracle.scan_complex_backward(lam, xc, g.astype(np.complex64), x0.astype(np.complex64))
    np.testing.assert_allclose(gu.real, gb, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(gu.imag, 0.0)
    np.testing.assert_allclose(glam.real, ga.sum(axis=(0, 1)), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gxc0.real, gx0, rtol=1e-12, atol=1e-13)


def test_backward_empty_and_single_step():
    a, b, g, x0 = _real_case(8, T=1)
    x = oracle.scan_real(a, b, x0)
    ga, gb, gx0 = oracle.scan_real_backward(a, x, g, x0)
    np.testing.assert_array_equal(gb, g.astype(np.float64))
    np.testing.assert_allclose(ga[:, 0], g[:, 0].astype(np.float64) * x0, rtol=1e-15)
    np.testing.assert_allclose(gx0, a[:, 0].astype(np.float64) * g[:, 0], rtol=1e-15)
    e = np.zeros((2, 0, 3), np.float32)
    ga, gb, gx0 = oracle.scan_real_backward(e, e.astype(np.float64), e, x0)
    assert ga.shape == (2, 0, 3) and np.all(gx0 == 0.0)


def test_initial_state_gradient_without_x0():
    # The gradient of a zero initial state is still a_0 gb_0 (conj(lam) gu_0).
    a, b, g, _ = _real_case(9)
    x = oracle.scan_real(a, b)
    _, gb, gx0 = oracle.scan_real_backward(a, x, g, want_gx0=True)
    np.testing.assert_allclose(gx0, a[:, 0].astype(np.float64) * gb[:, 0], rtol=1e-15)
    lam, u, gc, _ = _cplx_case(10)
    xc = oracle.scan_complex(lam, u)
    _, gu, gc0 = oracle.scan_complex_backward(lam, xc, gc, want_gx0=True)
    np.testing.assert_allclose(gc0, np.conj(lam.astype(np.complex128)) * gu[:, 0], rtol=1e-15)
