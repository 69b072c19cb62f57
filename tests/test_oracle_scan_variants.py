"""Pins of the fused scan variants' oracle: minGRU and minLSTM from gate pre-activations
(minGRU page, minGRU and minLSTM sections), the real scan with one decay per channel (an
SLRU, LRU write-up, section on RWKV) and the LRU's normalised input (LRU write-up,
initialisation section).

Each is pinned by what the pages and the mathematics fix independently of the oracle's
loop: limits of the gates, convexity of the gated update, an equivalence between minLSTM
and minGRU, the unrolled sums of the scan form, and the stationary variance law that the
LRU's normalisation is there to give.
"""

import math

import numpy as np

import oracle
from linear_recurrence_rnn_amd import workloads

import brute


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def sig64(k):
    return 1.0 / (1.0 + np.exp(-np.asarray(k, np.float64)))


# ---- minGRU ----------------------------------------------------------------------

def test_mingru_gate_limits():
    h, x0 = rnd((2, 20, 4), 1), rnd((2, 4), 2)
    k_open = np.full(h.shape, 40.0, np.float32)    # z = 1: the state is the candidate
    np.testing.assert_allclose(oracle.scan_mingru(k_open, h, x0), h.astype(np.float64), rtol=0, atol=1e-15)
    k_shut = np.full(h.shape, -40.0, np.float32)   # z = 0: the state keeps x0
    np.testing.assert_allclose(oracle.scan_mingru(k_shut, h, x0), np.broadcast_to(x0[:, None, :], h.shape),
                               rtol=0, atol=1e-15)


def test_mingru_is_a_convex_combination():
    kz, h, x0 = rnd((3, 50, 5), 3, 2.0), rnd((3, 50, 5), 4), rnd((3, 5), 5)
    x = oracle.scan_mingru(kz, h, x0)
    seen = np.concatenate([x0[:, None, :], h], axis=1).astype(np.float64)
    lo, hi = np.minimum.accumulate(seen, axis=1)[:, 1:], np.maximum.accumulate(seen, axis=1)[:, 1:]
    assert np.all(x >= lo - 1e-12) and np.all(x <= hi + 1e-12)


def test_mingru_unrolled_sums():
    kz, h, x0 = rnd((2, 30, 3), 6, 1.5), rnd((2, 30, 3), 7), rnd((2, 3), 8)
    z = sig64(kz)
    ref = brute.scan_real_sums(1.0 - z, z * h.astype(np.float64), x0.astype(np.float64))
    np.testing.assert_allclose(oracle.scan_mingru(kz, h, x0), ref, rtol=1e-12, atol=1e-13)


# ---- minLSTM ---------------------------------------------------------------------

def test_minlstm_equal_gates_average():
    k, h, x0 = rnd((2, 25, 4), 9, 2.0), rnd((2, 25, 4), 10), rnd((2, 4), 11)
    ref = brute.scan_real_sums(np.full(h.shape, 0.5), 0.5 * h.astype(np.float64), x0.astype(np.float64))
    np.testing.assert_allclose(oracle.scan_minlstm(k, k, h, x0), ref, rtol=1e-13, atol=1e-14)


def test_minlstm_gate_limits():
    h, x0 = rnd((2, 20, 4), 12), rnd((2, 4), 13)
    hi, lo = np.full(h.shape, 40.0, np.float32), np.full(h.shape, -40.0, np.float32)
    # forget gate open, input gate shut: the state keeps x0; and the reverse: the candidate
    np.testing.assert_allclose(oracle.scan_minlstm(hi, lo, h, x0), np.broadcast_to(x0[:, None, :], h.shape),
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.scan_minlstm(lo, hi, h, x0), h.astype(np.float64), rtol=0, atol=1e-15)


def test_minlstm_is_mingru_with_the_log_ratio_gate():
    """i' = i / (f + i) = sigmoid(log i - log f): minLSTM is minGRU whose gate logit is
    log sigmoid(ki) - log sigmoid(kf)."""
    kf, ki, h, x0 = rnd((2, 40, 6), 14, 2.0), rnd((2, 40, 6), 15, 2.0), rnd((2, 40, 6), 16), rnd((2, 6), 17)
    kz = (np.log(sig64(ki)) - np.log(sig64(kf))).astype(np.float32)
    # kz is rounded to float32, so the two agree to float32 precision of the gate only.
    np.testing.assert_allclose(oracle.scan_minlstm(kf, ki, h, x0), oracle.scan_mingru(kz, h, x0),
                               rtol=2e-6, atol=2e-6)


# ---- real scan with one decay per channel ---------------------------------------

def test_real_decay_special_cases():
    u, x0 = rnd((2, 30, 3), 18), rnd((2, 3), 19)
    ones = np.ones(3, np.float32)
    np.testing.assert_allclose(oracle.scan_real_decay(ones, u, x0),
                               x0[:, None, :].astype(np.float64) + np.cumsum(u.astype(np.float64), axis=1),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(oracle.scan_real_decay(0 * ones, u, x0), u.astype(np.float64))


def test_real_decay_unrolled_sums():
    lam = np.random.default_rng(20).uniform(-1, 1, 5).astype(np.float32)
    u, x0 = rnd((3, 40, 5), 21), rnd((3, 5), 22)
    a = np.broadcast_to(lam.astype(np.float64), u.shape)
    np.testing.assert_allclose(oracle.scan_real_decay(lam, u, x0), brute.scan_real_sums(a, u.astype(np.float64),
                               x0.astype(np.float64)), rtol=1e-12, atol=1e-13)


# ---- LRU with normalised input ---------------------------------------------------

def test_complex_normalized_unrolled_sums():
    lr = workloads.make_lru(2, 30, 4, 23, 0.5, 0.99, math.pi)
    gamma = np.sqrt(1.0 - np.abs(lr["lam"].astype(np.complex128)) ** 2)
    x0 = (rnd((2, 4), 24) + 1j * rnd((2, 4), 25)).astype(np.complex64)
    ref = brute.scan_complex_sums(lr["lam"], gamma * lr["u"].astype(np.complex128), x0)
    np.testing.assert_allclose(oracle.scan_complex_normalized(lr["lam"], lr["u"], x0), ref, rtol=1e-11, atol=1e-12)


def test_complex_normalized_on_the_unit_circle():
    """r = 1, the end of the LRU write-up's range r in [0, 1]: gamma = 0, so the state only
    rotates x0, x_t = lam^{t+1} x0.  A unit-modulus lambda stored as complex64 has |lam|^2
    a rounding above or below 1; above (and at 1 exactly) the state is that rotation and
    finite, below it gamma is the small sqrt(1 - |lam|^2) of the unrolled sums."""
    lr = workloads.make_lru(2, 40, 64, 27, 1.0, 1.0, 2 * math.pi, with_x0=True)
    lam = lr["lam"].copy()
    lam[:4] = np.array([1, -1, 1j, -1j], dtype=np.complex64)
    m2 = lam.real.astype(np.float64) ** 2 + lam.imag.astype(np.float64) ** 2  # exact squares, one rounding
    edge = m2 >= 1.0
    assert edge.sum() >= 16 and (m2 > 1.0).sum() >= 8 and (~edge).sum() >= 8
    x = oracle.scan_complex_normalized(lam, lr["u"], lr["x0"])
    assert np.all(np.isfinite(x))
    rot = brute.scan_complex_sums(lam, np.zeros(lr["u"].shape, np.complex128), lr["x0"])
    np.testing.assert_allclose(x[..., edge], rot[..., edge], rtol=1e-12, atol=1e-13)
    gamma = np.sqrt(1.0 - m2[~edge])
    inner = brute.scan_complex_sums(lam[~edge], gamma * lr["u"][..., ~edge].astype(np.complex128),
                                    lr["x0"][:, ~edge])
    np.testing.assert_allclose(x[..., ~edge], inner, rtol=1e-9, atol=1e-10)


def test_complex_normalized_keeps_unit_variance():
    """White input of unit variance: the normalised state has unit variance once the start
    is forgotten (the raw one has 1 / (1 - |lam|^2)); 64 x 32 sequences, 5% tolerance."""
    B, T, C = 64, 400, 32
    lr = workloads.make_lru(B, T, C, 26, 0.5, 0.9, math.pi)
    x = oracle.scan_complex_normalized(lr["lam"], lr["u"])
    var = np.mean(np.abs(x[:, -50:]) ** 2)
    assert abs(var - 1.0) < 0.05
    raw = oracle.scan_complex(lr["lam"], lr["u"])
    assert np.mean(np.abs(raw[:, -50:]) ** 2) > 1.3
    # lambda = 0: gamma = 1 and the state is the input
    zero = np.zeros(C, np.complex64)
    np.testing.assert_allclose(oracle.scan_complex_normalized(zero, lr["u"][:2]), lr["u"][:2].astype(np.complex128),
                               rtol=0, atol=0)
