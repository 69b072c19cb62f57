"""Pins of the oracle's conditioning sums for dL/dw and dL/du (``oracle.wkv4_backward_cond``).

The GPU tests hold each channel of dL/dw and dL/du to its own tolerance, floored by the
magnitudes of the products its terms are made of (chain rule of eq. (14) of the RWKV-LLM
page, "Time-mixing block"; the gate of eq. (15); a carried state as in the page's
"并行训练和序列解码").  Those magnitude sums are pinned here by
  * brute force: every A'_t, |A'|_t, B'_t, B_t, A_t written out as its O(T^2) sum over the
    earlier steps, in float64, with and without the gate and a carried state;
  * the triangle inequality: |dL/dw_c| <= cw_c and |dL/du_c| <= cu_c;
  * agreement of the gradients returned alongside with ``wkv4_backward_ex``.
"""

import numpy as np

import brute
import oracle


def _rand(B, T, C, seed):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-3, 1, C)).astype(np.float32)
    u = (rng.standard_normal(C) * 0.5).astype(np.float32)
    k = rng.standard_normal((B, T, C)).astype(np.float32)
    v = rng.standard_normal((B, T, C)).astype(np.float32)
    gy = rng.standard_normal((B, T, C)).astype(np.float32)
    r = (rng.standard_normal((B, T, C)) * 2).astype(np.float32)
    s_in = np.stack([rng.standard_normal((B, C)), rng.uniform(0.2, 3.0, (B, C)), rng.uniform(-2.0, 2.0, (B, C))],
                    axis=-1).astype(np.float32)
    gs_out = rng.standard_normal((B, C, 2)).astype(np.float32)
    return w, u, k, v, gy, r, s_in, gs_out


def test_cond_brute_force_plain_and_gated():
    w, u, k, v, gy, r, _, _ = _rand(2, 9, 4, 11)
    for rr in (None, r):
        got = oracle.wkv4_backward_cond(w, u, k, v, gy, r=rr)
        gw, gu, cw, cu, _ = brute.wkv4_cond_sums(w, u, k, v, gy, r=rr)
        np.testing.assert_allclose(got[0], gw, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(got[1], gu, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(got[6], cw, rtol=1e-10)
        np.testing.assert_allclose(got[7], cu, rtol=1e-10)


def test_cond_brute_force_carried_state():
    # s_out is the state after the last token in the natural-log convention (a', b', p'),
    # here taken with p' = 0: dL/dA_T = gs_out[0], dL/dB_T = gs_out[1].
    w, u, k, v, gy, _, s_in, gs_out = _rand(2, 7, 3, 12)
    _, _, _, _, s_out = brute.wkv4_cond_sums(w, u, k, v, gy, s_in=s_in)
    s_out = s_out.astype(np.float32)
    got = oracle.wkv4_backward_cond(w, u, k, v, gy, s_in=s_in, s_out=s_out, gs_out=gs_out)
    gw, gu, cw, cu, _ = brute.wkv4_cond_sums(w, u, k, v, gy, s_in=s_in, gs_out=gs_out)
    np.testing.assert_allclose(got[0], gw, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(got[1], gu, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(got[6], cw, rtol=1e-9)
    np.testing.assert_allclose(got[7], cu, rtol=1e-9)


def test_cond_bounds_the_sums_and_matches_backward_ex():
    w, u, k, v, gy, r, s_in, gs_out = _rand(3, 40, 6, 13)
    s_out = np.stack([np.ones((3, 6)), np.full((3, 6), 2.0), np.zeros((3, 6))], axis=-1).astype(np.float32)
    for kw in ({}, {"r": r}, {"s_in": s_in, "s_out": s_out, "gs_out": gs_out}):
        got = oracle.wkv4_backward_cond(w, u, k, v, gy, **kw)
        ref = oracle.wkv4_backward_ex(w, u, k, v, gy, **kw)
        for i in range(4):
            np.testing.assert_array_equal(got[i], ref[i])
        assert np.all(np.abs(got[0]) <= got[6]) and np.all(np.abs(got[1]) <= got[7])
        assert np.all(got[6] > 0) and np.all(got[7] > 0)
