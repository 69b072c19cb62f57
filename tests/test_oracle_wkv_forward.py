"""Pins of the fp64 WKV-4 forward oracle against things other than itself.

Sources (RWKV-LLM page = "RWKV：基于RNN的LLM"; LRU write-up = the zzfmdn.com blog on
"Resurrecting Recurrent Neural Networks for Long Sequences"):
  * brute force of the sums of eq. (14) (RWKV-LLM page, "Time-mixing block");
  * the two-SLRU ratio in the LRU write-up's section on RWKV, with lam = e^{-w}, g = e^{u};
  * AFT, eqs. (9)-(10) of the RWKV-LLM page ("Transformers和AFT"), which eq. (14) equals
    when u = w;
  * closed forms and invariants that follow from eq. (14) with w >= 0 (eq. (10)'s remark).
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import brute
import oracle
from linear_recurrence_rnn_amd import workloads


def _rand(B, T, C, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-3, 1, C)).astype(np.float32)
    u = (rng.standard_normal(C) * 0.5).astype(np.float32)
    k = (rng.standard_normal((B, T, C)) * kscale).astype(np.float32)
    v = rng.standard_normal((B, T, C)).astype(np.float32)
    return w, u, k, v


def test_workload1_matches_brute_force():
    d = workloads.make_inputs(1)
    y = oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])
    ref = brute.wkv4_sums(d["w"], d["u"], d["k"], d["v"])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


@settings(max_examples=40, deadline=None)
@given(B=st.integers(1, 3), T=st.integers(1, 40), C=st.integers(1, 7),
       seed=st.integers(0, 2**31 - 1), kscale=st.sampled_from([0.5, 1.0, 4.0, 30.0]))
def test_brute_force_random_shapes(B, T, C, seed, kscale):
    w, u, k, v = _rand(B, T, C, seed, kscale)
    y = oracle.wkv4_forward(w, u, k, v)
    ref = brute.wkv4_sums(w, u, k, v)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_two_slru_form():
    w, u, k, v = _rand(2, 50, 6, 7)
    y = oracle.wkv4_forward(w, u, k, v)
    np.testing.assert_allclose(y, brute.wkv4_two_slru(w, u, k, v), rtol=1e-11, atol=1e-12)


def test_u_equal_w_is_aft_with_linear_decay():
    w, _, k, v = _rand(2, 40, 5, 11)
    y = oracle.wkv4_forward(w, w, k, v)
    np.testing.assert_allclose(y, brute.aft_decay(w, k, v), rtol=1e-11, atol=1e-12)


def test_u_not_w_differs_from_aft():
    # Guards against a decay exponent of -(t-i)w in the past sum (eq. (10)'s form):
    # with u != w the two definitions must differ.
    w, u, k, v = _rand(1, 20, 4, 12)
    y = oracle.wkv4_forward(w, u, k, v)
    assert np.max(np.abs(y - brute.aft_decay(w, k, v))) > 1e-3


def test_first_step_is_v0():
    w, u, k, v = _rand(3, 17, 9, 3, kscale=5.0)
    y = oracle.wkv4_forward(w, u, k, v)
    # y_0 = (beta v_0) / beta: v_0 up to two roundings.
    np.testing.assert_allclose(y[:, 0, :], v[:, 0, :].astype(np.float64), rtol=4e-16, atol=0)


def test_constant_v_and_convex_bounds():
    w, u, k, _ = _rand(2, 64, 8, 5, kscale=3.0)
    v = np.full(k.shape, -1.75, np.float32)
    y = oracle.wkv4_forward(w, u, k, v)
    np.testing.assert_allclose(y, -1.75, rtol=1e-14)
    # Positive weights: y_t is a convex combination of v_0..v_t.
    w, u, k, v = _rand(2, 64, 8, 6, kscale=3.0)
    y = oracle.wkv4_forward(w, u, k, v)
    lo = np.minimum.accumulate(v.astype(np.float64), axis=1)
    hi = np.maximum.accumulate(v.astype(np.float64), axis=1)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)


@pytest.mark.parametrize("u0", [0.0, 0.7, -1.3])
def test_zero_k_zero_w_closed_form(u0):
    # k = 0, w = 0: y_t = (sum_{i<t} v_i + e^u v_t) / (t + e^u); u = 0 is the running mean.
    B, T, C = 2, 30, 3
    rng = np.random.default_rng(1)
    v = rng.standard_normal((B, T, C)).astype(np.float32)
    k = np.zeros((B, T, C), np.float32)
    w = np.zeros(C, np.float32)
    u = np.full(C, u0, np.float32)
    y = oracle.wkv4_forward(w, u, k, v)
    vd = v.astype(np.float64)
    past = np.concatenate([np.zeros((B, 1, C)), np.cumsum(vd, axis=1)[:, :-1]], axis=1)
    t = np.arange(T)[None, :, None]
    g = np.exp(np.float64(np.float32(u0)))
    np.testing.assert_allclose(y, (past + g * vd) / (t + g), rtol=1e-13)
    if u0 == 0.0:
        np.testing.assert_allclose(y, np.cumsum(vd, axis=1) / (t + 1), rtol=1e-13)


def test_large_u_gives_v():
    w, _, k, v = _rand(2, 25, 4, 8)
    u = np.full(4, 60.0, np.float32)
    y = oracle.wkv4_forward(w, u, k, v)
    # The deviation from v_t is about B_t / e^{60+k_t} ~ 1e-24: below double rounding.
    np.testing.assert_allclose(y, v, rtol=1e-14, atol=1e-14)


def test_huge_w_gives_two_token_mix():
    # eps = e^{-w} -> 0 keeps only the newest past token i = t-1 (exponent 0).
    w, u, k, v = _rand(2, 30, 5, 9)
    w = np.full(5, 1e4, np.float32)
    y = oracle.wkv4_forward(w, u, k, v)
    kd, vd, ud = k.astype(np.float64), v.astype(np.float64), u.astype(np.float64)
    a = np.exp(kd[:, :-1])
    c = np.exp(ud + kd[:, 1:])
    mix = (a * vd[:, :-1] + c * vd[:, 1:]) / (a + c)
    np.testing.assert_allclose(y[:, 1:], mix, rtol=1e-13)
    np.testing.assert_allclose(y[:, 0], vd[:, 0], rtol=4e-16, atol=0)


def test_shift_k_and_affine_v():
    w, u, k, v = _rand(2, 40, 6, 10)
    # Dyadic grid so that k + 3.5 and 2 v + 0.25 are exact in float32.
    k = (np.round(k * 1024) / 1024).astype(np.float32)
    v = (np.round(v * 1024) / 1024).astype(np.float32)
    y = oracle.wkv4_forward(w, u, k, v)
    y2 = oracle.wkv4_forward(w, u, (k + np.float32(3.5)).astype(np.float32), v)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-13)
    v2 = (np.float32(2.0) * v + np.float32(0.25)).astype(np.float32)
    y3 = oracle.wkv4_forward(w, u, k, v2)
    np.testing.assert_allclose(y3, 2.0 * y + 0.25, rtol=1e-12, atol=1e-12)


def test_large_k_spread_is_stable():
    # Spikes of +-150 in k: e^{150} overflows float32 but the rescaled fp64 sums are fine.
    w, u, k, v = _rand(1, 40, 4, 13)
    k[0, 7, :] = 150.0
    k[0, 20, 1] = -150.0
    y = oracle.wkv4_forward(w, u, k, v)
    np.testing.assert_allclose(y, brute.wkv4_sums(w, u, k, v), rtol=1e-11, atol=1e-12)


def test_empty_shapes():
    for shape in [(0, 5, 3), (2, 0, 3), (2, 5, 0)]:
        B, T, C = shape
        y = oracle.wkv4_forward(np.ones(C, np.float32), np.zeros(C, np.float32),
                                np.zeros(shape, np.float32), np.zeros(shape, np.float32))
        assert y.shape == shape
