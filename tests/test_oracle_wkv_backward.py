"""Pins of the fp64 WKV-4 backward oracle.

The pages print no backward pass; the oracle applies the chain rule to eq. (14) of the
RWKV-LLM page ("RWKV：基于RNN的LLM", "Time-mixing block").  It is pinned by
  * central finite differences of the (separately pinned) forward oracle;
  * torch.autograd in float64 through the dense T x T evaluation of eq. (14);
  * the identities implied by eq. (14): shifting every k of one sequence leaves y
    unchanged, so sum_t dL/dk_t = 0; adding c to every v adds c to every y, so
    sum_s dL/dv_s = sum_t dL/dy_t.
"""

import numpy as np
import pytest

import brute
import oracle


def _rand(B, T, C, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-3, 1, C)).astype(np.float32)
    u = (rng.standard_normal(C) * 0.5).astype(np.float32)
    k = (rng.standard_normal((B, T, C)) * kscale).astype(np.float32)
    v = rng.standard_normal((B, T, C)).astype(np.float32)
    gy = rng.standard_normal((B, T, C)).astype(np.float32)
    return w, u, k, v, gy


def _loss_fd(w, u, k, v, gy):
    """Loss sum(gy * y) evaluated by the forward oracle on float64 copies."""
    return float(np.sum(gy.astype(np.float64) * _fwd64(w, u, k, v)))


def _fwd64(w, u, k, v):
    # The oracle reads float32; finite differences need float64 perturbations, so use
    # the brute-force sums (pinned to the oracle at rtol 1e-10 in the forward tests).
    return brute.wkv4_sums(w, u, k, v)


def test_against_torch_autograd():
    torch = pytest.importorskip("torch")
    w, u, k, v, gy = _rand(2, 24, 5, 1, kscale=2.0)
    gw, gu, gk, gv = oracle.wkv4_backward(w, u, k, v, gy)
    tw = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    tu = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    y = brute.wkv4_torch(tw, tu, tk, tv)
    (y * torch.tensor(gy, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(gw, tw.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gu, tu.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_against_finite_differences():
    w, u, k, v, gy = _rand(1, 12, 3, 2)
    w64, u64, k64, v64 = (x.astype(np.float64) for x in (w, u, k, v))
    gw, gu, gk, gv = oracle.wkv4_backward(w, u, k, v, gy)
    h = 1e-6

    def num(arr_name, idx):
        args = {"w": w64.copy(), "u": u64.copy(), "k": k64.copy(), "v": v64.copy()}
        args[arr_name][idx] += h
        lp = _loss_fd(args["w"], args["u"], args["k"], args["v"], gy)
        args[arr_name][idx] -= 2 * h
        lm = _loss_fd(args["w"], args["u"], args["k"], args["v"], gy)
        return (lp - lm) / (2 * h)

    for c in range(3):
        assert abs(num("w", (c,)) - gw[c]) < 1e-7 * max(1.0, abs(gw[c]))
        assert abs(num("u", (c,)) - gu[c]) < 1e-7 * max(1.0, abs(gu[c]))
    for idx in [(0, 0, 0), (0, 5, 1), (0, 11, 2), (0, 7, 0)]:
        assert abs(num("k", idx) - gk[idx]) < 1e-7 * max(1.0, abs(gk[idx]))
        assert abs(num("v", idx) - gv[idx]) < 1e-7 * max(1.0, abs(gv[idx]))


@pytest.mark.parametrize("kscale", [1.0, 2.0, 20.0])
def test_shift_identities(kscale):
    w, u, k, v, gy = _rand(3, 50, 7, 3, kscale=kscale)
    _, _, gk, gv = oracle.wkv4_backward(w, u, k, v, gy)
    scale = np.sqrt(np.mean(gk ** 2)) * 50
    np.testing.assert_allclose(gk.sum(axis=1), 0.0, atol=1e-12 * scale)
    np.testing.assert_allclose(gv.sum(axis=1), gy.astype(np.float64).sum(axis=1),
                               rtol=1e-11, atol=1e-11)


def test_huge_w_has_no_w_gradient():
    # eps = e^{-w} underflows: dL/dw = -sum g (A' - y B') / D with A' = B' = 0.
    w, u, k, v, gy = _rand(2, 20, 4, 4)
    w[:] = 1e4
    gw, _, _, _ = oracle.wkv4_backward(w, u, k, v, gy)
    np.testing.assert_array_equal(gw, 0.0)


def test_single_step_closed_form():
    # T = 1: y_0 = v_0, so dL/dv_0 = gy_0 and every other gradient is zero.
    w, u, k, v, gy = _rand(2, 1, 5, 5)
    gw, gu, gk, gv = oracle.wkv4_backward(w, u, k, v, gy)
    np.testing.assert_allclose(gv, gy, rtol=1e-15)
    np.testing.assert_allclose(gk, 0.0, atol=1e-15)
    np.testing.assert_allclose(gu, 0.0, atol=1e-15)
    np.testing.assert_allclose(gw, 0.0, atol=1e-15)


def test_batch_sum_of_w_u_gradients():
    # gw and gu are sums over the batch of per-sequence contributions.
    w, u, k, v, gy = _rand(3, 16, 4, 6)
    gw, gu, _, _ = oracle.wkv4_backward(w, u, k, v, gy)
    parts = [oracle.wkv4_backward(w, u, k[b:b + 1], v[b:b + 1], gy[b:b + 1]) for b in range(3)]
    np.testing.assert_allclose(gw, sum(p[0] for p in parts), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gu, sum(p[1] for p in parts), rtol=1e-13, atol=1e-14)
