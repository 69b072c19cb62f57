"""Pins of the oracle's backward of the fused scan variants: minGRU and minLSTM from gate
pre-activations (minGRU page, minGRU and minLSTM sections), the real scan with one decay per
channel (LRU write-up, section on RWKV) and the LRU's normalised input (LRU write-up,
initialisation section).  The pages give no backward; each is the chain rule of the
forward reading.

Each pin is independent of the oracle's C loops: torch fp64 autograd of a plain torch
forward, central finite differences of that forward, the gates' limits with closed forms,
and the chain through the plain scan adjoint (itself pinned by autograd and the unrolled
sums) with the gates' derivatives.
"""

import math

import numpy as np
import pytest

import brute
import oracle
from linear_recurrence_rnn_amd import workloads

torch = pytest.importorskip("torch")


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def t64(x, grad=True):
    dt = torch.complex128 if np.iscomplexobj(x) else torch.float64
    return torch.tensor(x, dtype=dt, requires_grad=grad)


def sig64(k):
    return 1.0 / (1.0 + np.exp(-np.asarray(k, np.float64)))


def close(mine, ref, rtol=1e-11, atol=1e-12):
    np.testing.assert_allclose(mine, ref, rtol=rtol, atol=atol)


def lru_case(seed, B=2, T=11, C=3, r_lo=0.5, r_hi=0.99):
    rng = np.random.default_rng(seed)
    d = workloads.make_lru(B, T, C, seed, r_lo, r_hi, 2 * math.pi)
    g = (rng.standard_normal((B, T, C)) + 1j * rng.standard_normal((B, T, C))).astype(np.complex64)
    x0 = (rng.standard_normal((B, C)) + 1j * rng.standard_normal((B, C))).astype(np.complex64)
    return d["lam"], d["u"], g, x0


# ---- autograd ------------------------------------------------------------------------

@pytest.mark.parametrize("with_x0", [True, False])
def test_mingru_backward_matches_autograd(with_x0):
    kz, h, g = rnd((2, 13, 3), 1, 1.5), rnd((2, 13, 3), 2), rnd((2, 13, 3), 3)
    x0 = rnd((2, 3), 4) if with_x0 else None
    x = oracle.scan_mingru(kz, h, x0)
    gkz, gh, gx0 = oracle.scan_mingru_backward(kz, h, x, g, x0, want_gx0=True)
    tk, th = t64(kz), t64(h)
    tx0 = t64(x0) if with_x0 else t64(np.zeros((2, 3), np.float32))
    brute.mingru_torch(tk, th, tx0).backward(torch.tensor(g, dtype=torch.float64))
    close(gkz, tk.grad.numpy())
    close(gh, th.grad.numpy())
    close(gx0, tx0.grad.numpy())


@pytest.mark.parametrize("with_x0", [True, False])
def test_minlstm_backward_matches_autograd(with_x0):
    kf, ki, h, g = rnd((2, 13, 3), 5, 2.0), rnd((2, 13, 3), 6, 2.0), rnd((2, 13, 3), 7), rnd((2, 13, 3), 8)
    x0 = rnd((2, 3), 9) if with_x0 else None
    x = oracle.scan_minlstm(kf, ki, h, x0)
    gkf, gki, gh, gx0 = oracle.scan_minlstm_backward(kf, ki, h, x, g, x0, want_gx0=True)
    tf, ti, th = t64(kf), t64(ki), t64(h)
    tx0 = t64(x0) if with_x0 else t64(np.zeros((2, 3), np.float32))
    brute.minlstm_torch(tf, ti, th, tx0).backward(torch.tensor(g, dtype=torch.float64))
    close(gkf, tf.grad.numpy())
    close(gki, ti.grad.numpy())
    close(gh, th.grad.numpy())
    close(gx0, tx0.grad.numpy())


@pytest.mark.parametrize("with_x0", [True, False])
def test_real_decay_backward_matches_autograd(with_x0):
    lam = np.random.default_rng(10).uniform(-1, 1, 3).astype(np.float32)
    u, g = rnd((2, 13, 3), 11), rnd((2, 13, 3), 12)
    x0 = rnd((2, 3), 13) if with_x0 else None
    x = oracle.scan_real_decay(lam, u, x0)
    glam, gu, gx0 = oracle.scan_real_decay_backward(lam, x, g, x0, want_gx0=True)
    tl, tu = t64(lam), t64(u)
    tx0 = t64(x0) if with_x0 else t64(np.zeros((2, 3), np.float32))
    brute.scan_torch(tl, tu, tx0).backward(torch.tensor(g, dtype=torch.float64))
    close(glam, tl.grad.numpy())
    close(gu, tu.grad.numpy())
    close(gx0, tx0.grad.numpy())


@pytest.mark.parametrize("with_x0", [True, False])
def test_lru_normalized_backward_matches_autograd(with_x0):
    lam, u, g, x0 = lru_case(14)
    if not with_x0:
        x0 = None
    x = oracle.scan_complex_normalized(lam, u, x0)
    glam, gu, gx0 = oracle.scan_complex_normalized_backward(lam, u, x, g, x0, want_gx0=True)
    tl, tu = t64(lam), t64(u)
    tx0 = t64(x0) if with_x0 else t64(np.zeros((2, 3), np.complex64))
    brute.lru_normalized_torch(tl, tu, tx0).backward(torch.tensor(g, dtype=torch.complex128))
    close(glam, tl.grad.numpy(), rtol=1e-10, atol=1e-11)
    close(gu, tu.grad.numpy())
    close(gx0, tx0.grad.numpy())


def test_lru_normalized_backward_on_the_unit_circle():
    """r = 1 (gamma = 0, including complex64 lambdas whose |lam|^2 rounds above 1): nothing
    reaches u, and dL/dlambda and dL/dx0 are the plain complex scan's unrolled adjoint sums
    (gamma has no derivative there and its term is taken as 0); below 1 the gradients are
    torch autograd's of the plain torch forward."""
    B, T, C = 2, 30, 48
    lr = workloads.make_lru(B, T, C, 31, 1.0, 1.0, 2 * math.pi, with_x0=True)
    lam = lr["lam"].copy()
    lam[:4] = np.array([1, -1, 1j, -1j], dtype=np.complex64)
    m2 = lam.real.astype(np.float64) ** 2 + lam.imag.astype(np.float64) ** 2  # exact squares, one rounding
    edge = m2 >= 1.0
    assert (m2 > 1.0).sum() >= 8 and (~edge).sum() >= 8
    g = (rnd((B, T, C), 32) + 1j * rnd((B, T, C), 33)).astype(np.complex64)
    x = oracle.scan_complex_normalized(lam, lr["u"], lr["x0"])
    glam, gu, gx0 = oracle.scan_complex_normalized_backward(lam, lr["u"], x, g, lr["x0"], want_gx0=True)
    assert np.all(np.isfinite(glam)) and np.all(np.isfinite(gu)) and np.all(np.isfinite(gx0))
    assert np.all(gu[..., edge] == 0)
    rl, _, r0 = brute.scan_complex_backward_sums(lam[edge], g[..., edge], x[..., edge], lr["x0"][:, edge])
    close(glam[edge], rl, rtol=1e-10, atol=1e-10)
    close(gx0[:, edge], r0, rtol=1e-11, atol=1e-11)
    tl, tu, tx0 = t64(lam[~edge]), t64(lr["u"][..., ~edge]), t64(lr["x0"][:, ~edge])
    brute.lru_normalized_torch(tl, tu, tx0).backward(torch.tensor(g[..., ~edge], dtype=torch.complex128))
    # Just below 1, 1 - |lam|^2 cancels to ~1e-8, so torch's |lam| (a square root, then
    # squared) and the oracle's exact |lam|^2 give gamma's -lam/gamma term to ~1e-8 only.
    close(glam[~edge], tl.grad.numpy(), rtol=1e-7, atol=1e-9)
    close(gu[..., ~edge], tu.grad.numpy(), rtol=1e-7, atol=1e-12)
    close(gx0[:, ~edge], tx0.grad.numpy())


# ---- finite differences of the plain forward ---------------------------------------

def test_minlstm_backward_finite_differences():
    """Central differences of the torch forward (float64) at a few entries of each input."""
    kf, ki, h, g = rnd((1, 9, 2), 15, 2.0), rnd((1, 9, 2), 16, 2.0), rnd((1, 9, 2), 17), rnd((1, 9, 2), 18)
    x0 = rnd((1, 2), 19)
    x = oracle.scan_minlstm(kf, ki, h, x0)
    grads = oracle.scan_minlstm_backward(kf, ki, h, x, g, x0)
    args = [kf.astype(np.float64), ki.astype(np.float64), h.astype(np.float64)]

    def loss(a):
        with torch.no_grad():
            y = brute.minlstm_torch(*(torch.tensor(z) for z in a), torch.tensor(x0, dtype=torch.float64))
        return float((y * torch.tensor(g, dtype=torch.float64)).sum())

    eps = 1e-6
    for which in range(3):
        for idx in [(0, 0, 0), (0, 4, 1), (0, 8, 0)]:
            up = [z.copy() for z in args]
            dn = [z.copy() for z in args]
            up[which][idx] += eps
            dn[which][idx] -= eps
            fd = (loss(up) - loss(dn)) / (2 * eps)
            assert abs(fd - grads[which][idx]) <= 1e-7 * max(1.0, abs(fd))


# ---- limits and closed forms -------------------------------------------------------

def test_mingru_backward_open_and_shut_gates():
    h, g, x0 = rnd((2, 10, 3), 20), rnd((2, 10, 3), 21), rnd((2, 3), 22)
    # z = 1: x_t = h_t, so dL/dh = g exactly, nothing reaches x0, and the gate's slope is 0.
    k_open = np.full(h.shape, 40.0, np.float32)
    x = oracle.scan_mingru(k_open, h, x0)
    gkz, gh, gx0 = oracle.scan_mingru_backward(k_open, h, x, g, x0)
    close(gh, g.astype(np.float64), rtol=1e-15, atol=1e-15)
    close(gx0, np.zeros((2, 3)), atol=1e-15)
    assert np.max(np.abs(gkz)) < 1e-15
    # z = 0: x_t = x0 for every t, so dL/dx0 is the sum of the gradients over time.
    k_shut = -k_open
    x = oracle.scan_mingru(k_shut, h, x0)
    gkz, gh, gx0 = oracle.scan_mingru_backward(k_shut, h, x, g, x0)
    close(gx0, g.astype(np.float64).sum(axis=1), rtol=1e-12, atol=1e-13)
    assert np.max(np.abs(gh)) < 1e-15


def test_real_decay_backward_limits():
    u, g, x0 = rnd((2, 10, 3), 23), rnd((2, 10, 3), 24), rnd((2, 3), 25)
    ones = np.ones(3, np.float32)
    x = oracle.scan_real_decay(ones, u, x0)
    glam, gu, gx0 = oracle.scan_real_decay_backward(ones, x, g, x0)
    # lam = 1: dL/du_t is the reverse cumulative sum of the gradients.
    close(gu, np.cumsum(g[:, ::-1].astype(np.float64), axis=1)[:, ::-1], rtol=1e-13, atol=1e-13)
    zeros = np.zeros(3, np.float32)
    x = oracle.scan_real_decay(zeros, u, x0)
    glam, gu, gx0 = oracle.scan_real_decay_backward(zeros, x, g, x0)
    # lam = 0: x = u, so dL/du = g, and dL/dlam = sum over b, t of g_t x_{t-1} with x_{-1} = x0.
    close(gu, g.astype(np.float64), rtol=0, atol=0)
    xp = np.concatenate([x0[:, None, :].astype(np.float64), u[:, :-1].astype(np.float64)], axis=1)
    close(glam, (g.astype(np.float64) * xp).sum(axis=(0, 1)), rtol=1e-12, atol=1e-13)
    close(gx0, np.zeros((2, 3)), atol=0)


# ---- chain through the plain scan adjoints --------------------------------------------

def test_gated_backwards_chain_through_the_real_scan_adjoint():
    """minGRU and minLSTM are the real scan with a = 1 - z (f') and b = z h (i' h): their
    gradients are the plain adjoint's (ga, gb) times the gates' derivatives."""
    kz, h, g, x0 = rnd((2, 12, 3), 26, 2.0), rnd((2, 12, 3), 27), rnd((2, 12, 3), 28), rnd((2, 3), 29)
    z = sig64(kz)
    x = oracle.scan_mingru(kz, h, x0)
    ga, gb, gx0r = oracle.scan_real_backward((1.0 - z).astype(np.float32), x, g, x0)
    gkz, gh, gx0 = oracle.scan_mingru_backward(kz, h, x, g, x0)
    # a = 1 - z was rounded to float32 for the plain adjoint's carry: compare loosely.
    close(gkz, (gb * h - ga) * z * (1.0 - z), rtol=1e-6, atol=1e-7)
    close(gh, gb * z, rtol=1e-6, atol=1e-7)
    close(gx0, gx0r, rtol=1e-6, atol=1e-7)

    kf, ki = rnd((2, 12, 3), 30, 2.0), rnd((2, 12, 3), 31, 2.0)
    f, i = sig64(kf), sig64(ki)
    a = f / (f + i)
    x = oracle.scan_minlstm(kf, ki, h, x0)
    ga, gb, _ = oracle.scan_real_backward(a.astype(np.float32), x, g, x0)
    gkf, gki, gh, _ = oracle.scan_minlstm_backward(kf, ki, h, x, g, x0)
    da = ga - gb * h  # dL/da with b = (1 - a) h
    close(gkf, da * a * (1.0 - a) * (1.0 - f), rtol=1e-6, atol=1e-7)
    close(gki, -da * a * (1.0 - a) * (1.0 - i), rtol=1e-6, atol=1e-7)
    close(gh, gb * (1.0 - a), rtol=1e-6, atol=1e-7)


def test_lru_normalized_backward_chains_the_complex_adjoint():
    """x = scan(lam, gamma u): dL/du = gamma times the plain adjoint's dL/du, and dL/dlam
    adds dL/dgamma dgamma/dlam = -(Re sum conj(gu) u / gamma) lam to the plain one."""
    lam, u, g, x0 = lru_case(32)
    gam = np.sqrt(1.0 - np.abs(lam.astype(np.complex128)) ** 2)
    x = oracle.scan_complex_normalized(lam, u, x0)
    glam_p, gu_p, gx0_p = oracle.scan_complex_backward(lam, x, g, x0)
    glam, gu, gx0 = oracle.scan_complex_normalized_backward(lam, u, x, g, x0)
    close(gu, gam * gu_p, rtol=1e-12, atol=1e-13)
    close(gx0, gx0_p, rtol=1e-12, atol=1e-13)
    dgam = np.real(np.conj(gu_p) * u.astype(np.complex128)).sum(axis=(0, 1))
    close(glam, glam_p - dgam / gam * lam.astype(np.complex128), rtol=1e-11, atol=1e-12)


def test_empty_sequence_gives_zero_gradients():
    kz = np.zeros((2, 0, 3), np.float32)
    x0 = rnd((2, 3), 33)
    gkz, gh, gx0 = oracle.scan_mingru_backward(kz, kz, np.zeros((2, 0, 3)), kz, x0)
    assert gkz.shape == (2, 0, 3) and np.all(gx0 == 0)
    glam, gu, gx0 = oracle.scan_real_decay_backward(np.ones(3, np.float32), np.zeros((2, 0, 3)), kz, x0)
    assert np.all(glam == 0) and np.all(gx0 == 0)
