"""Pins of the fp64 real and complex diagonal-scan oracles.

Sources: the minGRU page's scan form v_t = a_t (.) v_{t-1} + b_t ("Were RNNs All We
Needed?" news item, minGRU section) and the LRU write-up (zzfmdn.com blog on
"Resurrecting Recurrent Neural Networks for Long Sequences"): the element-wise complex
recurrence and its unrolled sum (eqs. lr-xx, lr-e), the cumsum form and the two-halves
split identity (parallelisation section), and the variance law (initialisation section).
"""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import brute
import oracle
from linear_recurrence_rnn_amd import workloads


def _lru(B, T, C, seed, r_lo=0.9, r_hi=0.999, theta_hi=math.pi / 10):
    return workloads.make_lru(B, T, C, seed, r_lo, r_hi, theta_hi)


@settings(max_examples=30, deadline=None)
@given(B=st.integers(1, 3), T=st.integers(1, 30), C=st.integers(1, 6),
       seed=st.integers(0, 2**31 - 1), with_x0=st.booleans())
def test_real_brute_force(B, T, C, seed, with_x0):
    rng = np.random.default_rng(seed)
    a = rng.uniform(-1.2, 1.2, (B, T, C)).astype(np.float32)
    b = rng.standard_normal((B, T, C)).astype(np.float32)
    x0 = rng.standard_normal((B, C)).astype(np.float32) if with_x0 else None
    np.testing.assert_allclose(oracle.scan_real(a, b, x0), brute.scan_real_sums(a, b, x0),
                               rtol=1e-11, atol=1e-12)


@settings(max_examples=30, deadline=None)
@given(B=st.integers(1, 3), T=st.integers(1, 30), C=st.integers(1, 6),
       seed=st.integers(0, 2**31 - 1), with_x0=st.booleans())
def test_complex_brute_force(B, T, C, seed, with_x0):
    d = _lru(B, T, C, seed, 0.5, 1.0, 2 * math.pi)
    rng = np.random.default_rng(seed + 1)
    x0 = None
    if with_x0:
        x0 = (rng.standard_normal((B, C)) + 1j * rng.standard_normal((B, C))).astype(np.complex64)
    np.testing.assert_allclose(oracle.scan_complex(d["lam"], d["u"], x0),
                               brute.scan_complex_sums(d["lam"], d["u"], x0),
                               rtol=1e-11, atol=1e-12)


def test_complex_cumsum_identity():
    d = _lru(2, 48, 5, 3)
    np.testing.assert_allclose(oracle.scan_complex(d["lam"], d["u"]),
                               brute.scan_complex_cumsum(d["lam"], d["u"]), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("split", [1, 17, 63])
def test_split_identity(split):
    # Scan [0, split), then continue from its last state over [split, T): same as one scan.
    d = _lru(2, 64, 4, 4)
    full = oracle.scan_complex(d["lam"], d["u"])
    first = oracle.scan_complex(d["lam"], d["u"][:, :split])
    x0 = first[:, -1].astype(np.complex64)
    second = oracle.scan_complex(d["lam"], d["u"][:, split:], x0)
    np.testing.assert_allclose(second, full[:, split:], rtol=2e-6, atol=2e-6)  # x0 rounded to c64
    rng = np.random.default_rng(5)
    a = rng.uniform(0, 1, (2, 64, 4)).astype(np.float32)
    b = rng.standard_normal((2, 64, 4)).astype(np.float32)
    full = oracle.scan_real(a, b)
    first = oracle.scan_real(a[:, :split], b[:, :split])
    second = oracle.scan_real(a[:, split:], b[:, split:], first[:, -1].astype(np.float32))
    np.testing.assert_allclose(second, full[:, split:], rtol=1e-6, atol=1e-6)


def test_real_special_cases():
    rng = np.random.default_rng(6)
    b = rng.standard_normal((3, 40, 5)).astype(np.float32)
    ones = np.ones_like(b)
    np.testing.assert_allclose(oracle.scan_real(ones, b), np.cumsum(b.astype(np.float64), axis=1),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(oracle.scan_real(np.zeros_like(b), b), b.astype(np.float64))
    x0 = rng.standard_normal((3, 5)).astype(np.float32)
    np.testing.assert_allclose(oracle.scan_real(ones, np.zeros_like(b), x0),
                               np.broadcast_to(x0[:, None, :], b.shape), rtol=0, atol=0)


def test_mingru_special_cases():
    # h_t = (1 - z_t) h_{t-1} + z_t h~_t: z = 1 gives h = h~, z = 0 keeps h_0 = 0.
    rng = np.random.default_rng(7)
    h = rng.standard_normal((2, 30, 4)).astype(np.float32)
    z = np.ones_like(h)
    np.testing.assert_array_equal(oracle.scan_real(1 - z, z * h), h.astype(np.float64))
    z = np.zeros_like(h)
    np.testing.assert_array_equal(oracle.scan_real(1 - z, z * h), 0.0)


def test_complex_zero_phase_is_real_scan():
    d = _lru(2, 50, 6, 8, theta_hi=0.0)
    lam = d["lam"]
    assert np.all(lam.imag == 0)
    u = d["u"]
    x = oracle.scan_complex(lam, u)
    a = np.broadcast_to(lam.real[None, None, :], u.shape).astype(np.float32)
    np.testing.assert_allclose(x.real, oracle.scan_real(a, u.real.copy()), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(x.imag, oracle.scan_real(a, u.imag.copy()), rtol=1e-14, atol=1e-14)


def test_complex_conjugation_and_linearity():
    d = _lru(2, 40, 5, 9)
    lam, u = d["lam"], d["u"]
    x = oracle.scan_complex(lam, u)
    np.testing.assert_allclose(oracle.scan_complex(np.conj(lam), np.conj(u)), np.conj(x),
                               rtol=1e-14, atol=1e-14)
    d2 = _lru(2, 40, 5, 10)
    x2 = oracle.scan_complex(lam, d2["u"])
    s = (u + d2["u"]).astype(np.complex64)  # rounding of the sum is part of the input
    np.testing.assert_allclose(oracle.scan_complex(lam, s), x + x2, rtol=1e-6, atol=1e-6)
    # A real scale by a power of two is exact.
    np.testing.assert_allclose(oracle.scan_complex(lam, (4 * u).astype(np.complex64)), 4 * x,
                               rtol=1e-14, atol=1e-14)


def test_lambda_power_impulse():
    # u = impulse at t = 0 gives x_t = lam^t.
    C = 6
    lam = _lru(1, 1, C, 11, 0.5, 1.0, 2 * math.pi)["lam"]
    u = np.zeros((1, 80, C), np.complex64)
    u[0, 0, :] = 1.0
    x = oracle.scan_complex(lam, u)
    t = np.arange(80)[:, None]
    np.testing.assert_allclose(x[0], lam.astype(np.complex128)[None, :] ** t, rtol=1e-12, atol=1e-14)


@pytest.mark.slow
def test_variance_law():
    # LRU write-up, initialisation section: E|x_t|^2 = (1 - r^{2(t+1)}) E|u|^2 / (1 - r^2)
    # for zero-mean i.i.d. u; here E|u|^2 = 1 (re, im ~ N(0, 1/2)).
    B, T, C = 8, 4096, 64
    d = _lru(B, T, C, 12)
    x = oracle.scan_complex(d["lam"], d["u"])
    r2 = np.abs(d["lam"].astype(np.complex128)) ** 2
    t = np.arange(T)[:, None]
    theory = (1 - r2[None, :] ** (t + 1)) / (1 - r2[None, :])  # r^{2(t+1)} = (r^2)^{t+1}
    ratio = np.mean(np.abs(x) ** 2, axis=0) / theory  # (T, C), mean over the batch
    assert abs(np.mean(ratio) - 1.0) < 0.05


def test_empty_shapes():
    for shape in [(0, 4, 2), (2, 0, 2), (2, 4, 0)]:
        z = np.zeros(shape, np.float32)
        assert oracle.scan_real(z, z).shape == shape
        lam = np.zeros(shape[2], np.complex64)
        assert oracle.scan_complex(lam, z.astype(np.complex64)).shape == shape
