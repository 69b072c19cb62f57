"""O(T^2) brute-force evaluations of the defining sums, used only to pin the oracle.

These are written directly from the printed sums, not from the recurrences the oracle
uses, so a mistake in the oracle's recurrence (a dropped term, an off-by-one decay
exponent, a swapped operand) shows up as a mismatch.
"""

from __future__ import annotations

import numpy as np


def wkv4_sums(w, u, k, v):
    """RWKV-LLM page, eq. (14), evaluated term by term for every (b, t, c).

    y_t = (sum_{i<t} e^{-(t-1-i)w+k_i} v_i + e^{u+k_t} v_t)
        / (sum_{i<t} e^{-(t-1-i)w+k_i}     + e^{u+k_t}).
    No rescaling: meant for tiny inputs with |k| well below 700.
    """
    w = np.asarray(w, np.float64)
    u = np.asarray(u, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, C = k.shape
    y = np.empty((B, T, C))
    for b in range(B):
        for c in range(C):
            for t in range(T):
                num = 0.0
                den = 0.0
                for i in range(t):
                    e = np.exp(-(t - 1 - i) * w[c] + k[b, i, c])
                    num += e * v[b, i, c]
                    den += e
                cur = np.exp(u[c] + k[b, t, c])
                y[b, t, c] = (num + cur * v[b, t, c]) / (den + cur)
    return y


def aft_decay(w, k, v):
    """RWKV-LLM page, eqs. (9)-(10): AFT with w_{t,i} = -(t-i) w, sums over i <= t."""
    w = np.asarray(w, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, C = k.shape
    y = np.empty((B, T, C))
    for t in range(T):
        i = np.arange(t + 1)
        e = np.exp(-(t - i)[None, :, None] * w[None, None, :] + k[:, : t + 1, :])
        y[:, t, :] = (e * v[:, : t + 1, :]).sum(1) / e.sum(1)
    return y


def wkv4_two_slru(w, u, k, v):
    """LRU write-up, section on RWKV: the ratio of two SLRU recurrences,

    x_t = (y_t + (g*lam - 1) e^{k_t} v_t) / (z_t + (g*lam - 1) e^{k_t}),
    y_t = lam y_{t-1} + e^{k_t} v_t,   z_t = lam z_{t-1} + e^{k_t},

    with lam = e^{-w} and g = e^{u} (the sigma(r) gate left out).
    """
    w = np.asarray(w, np.float64)
    u = np.asarray(u, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, C = k.shape
    lam = np.exp(-w)
    g = np.exp(u)
    ys = np.zeros((B, C))
    zs = np.zeros((B, C))
    out = np.empty((B, T, C))
    for t in range(T):
        ek = np.exp(k[:, t, :])
        ys = lam * ys + ek * v[:, t, :]
        zs = lam * zs + ek
        out[:, t, :] = (ys + (g * lam - 1.0) * ek * v[:, t, :]) / (zs + (g * lam - 1.0) * ek)
    return out


def wkv4_torch(w, u, k, v):
    """Eq. (14) as a dense masked T x T weighting in torch float64 (for autograd).

    w, u: (C,), k, v: (B,T,C) torch float64 tensors.
    """
    import torch

    B, T, C = k.shape
    t = torch.arange(T, dtype=torch.float64)
    dist = (t[:, None] - 1.0 - t[None, :])  # (t, i) -> t-1-i
    mask = (t[None, :] < t[:, None])  # i < t
    # expo[b, c, t, i] = -(t-1-i) w_c + k_{b,i,c}
    kk = k.permute(0, 2, 1)  # (B,C,T)
    vv = v.permute(0, 2, 1)
    expo = -dist[None, None] * w[None, :, None, None] + kk[:, :, None, :]
    expo = torch.where(mask[None, None], expo, torch.full_like(expo, -torch.inf))
    E = torch.exp(expo)
    cur = torch.exp(u[None, :, None] + kk)
    num = (E * vv[:, :, None, :]).sum(-1) + cur * vv
    den = E.sum(-1) + cur
    return (num / den).permute(0, 2, 1)


def scan_real_sums(a, b, x0=None):
    """x_t = sum_{k<=t} (prod_{j=k+1}^{t} a_j) b_k + (prod_{j=0}^{t} a_j) x0, term by term."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    B, T, C = a.shape
    x0 = np.zeros((B, C)) if x0 is None else np.asarray(x0, np.float64)
    x = np.empty((B, T, C))
    for t in range(T):
        acc = np.prod(a[:, : t + 1, :], axis=1) * x0
        for kk in range(t + 1):
            acc = acc + np.prod(a[:, kk + 1: t + 1, :], axis=1) * b[:, kk, :]
        x[:, t, :] = acc
    return x


def scan_complex_sums(lam, u, x0=None):
    """LRU write-up, eq. lr-xx unrolled: x_t = sum_{k<=t} lam^{t-k} u_k (+ lam^{t+1} x0)."""
    lam = np.asarray(lam, np.complex128)
    u = np.asarray(u, np.complex128)
    B, T, C = u.shape
    x0 = np.zeros((B, C), np.complex128) if x0 is None else np.asarray(x0, np.complex128)
    x = np.empty((B, T, C), np.complex128)
    for t in range(T):
        pw = lam[None, None, :] ** (t - np.arange(t + 1))[None, :, None]
        x[:, t, :] = (pw * u[:, : t + 1, :]).sum(1) + lam ** (t + 1) * x0
    return x


def scan_complex_cumsum(lam, u):
    """LRU write-up, parallelisation section: x_t = lam^t * cumsum_k(lam^{-k} u_k).

    Exact in real arithmetic; only usable for short sequences (lam^{-k} grows).
    """
    lam = np.asarray(lam, np.complex128)
    u = np.asarray(u, np.complex128)
    T = u.shape[1]
    t = np.arange(T)[None, :, None]
    return lam ** t * np.cumsum(lam ** (-t) * u, axis=1)


def scan_real_backward_sums(a, gx, x, x0=None):
    """Adjoint of the real scan by its unrolled sums: gb_t = sum_{s>=t} (prod_{k=t+1..s} a_k)
    gx_s, ga_t = gb_t x_{t-1}, gx0 = a_0 gb_0 (O(T^2), float64)."""
    a = np.asarray(a, np.float64)
    g = np.asarray(gx, np.float64)
    x = np.asarray(x, np.float64)
    B, T, C = a.shape
    gb = np.zeros((B, T, C))
    for t in range(T):
        prod = np.ones((B, C))
        for s in range(t, T):
            if s > t:
                prod = prod * a[:, s]
            gb[:, t] += prod * g[:, s]
    xprev = np.concatenate([(np.zeros((B, 1, C)) if x0 is None else np.asarray(x0, np.float64)[:, None]),
                            x[:, :-1]], axis=1)
    ga = gb * xprev
    gx0 = None if x0 is None else a[:, 0] * gb[:, 0]
    return ga, gb, gx0


def scan_complex_backward_sums(lam, gx, x, x0=None):
    """Adjoint of the complex scan by its unrolled sums: gu_t = sum_{s>=t} conj(lam)^{s-t}
    gx_s, glam = sum_{b,t} gu_t conj(x_{t-1}), gx0 = conj(lam) gu_0 (O(T^2), complex128)."""
    lc = np.conj(np.asarray(lam, np.complex128))
    g = np.asarray(gx, np.complex128)
    x = np.asarray(x, np.complex128)
    B, T, C = g.shape
    gu = np.zeros((B, T, C), np.complex128)
    for t in range(T):
        for s in range(t, T):
            gu[:, t] += lc ** (s - t) * g[:, s]
    xprev = np.concatenate([(np.zeros((B, 1, C), np.complex128) if x0 is None
                             else np.asarray(x0, np.complex128)[:, None]), x[:, :-1]], axis=1)
    glam = (gu * np.conj(xprev)).sum(axis=(0, 1))
    gx0 = None if x0 is None else lc * gu[:, 0]
    return glam, gu, gx0


def scan_torch(coef, inp, x0=None):
    """x_t = coef_t x_{t-1} + inp_t as a plain torch loop (real or complex; coef may be (C,)
    or (B,T,C)), differentiable by autograd."""
    import torch
    B, T, C = inp.shape
    s = torch.zeros((B, C), dtype=inp.dtype) if x0 is None else x0
    out = []
    for t in range(T):
        ct = coef if coef.dim() == 1 else coef[:, t]
        s = ct * s + inp[:, t]
        out.append(s)
    return torch.stack(out, dim=1)


def wkv4_state_torch(w, u, k, v, a0, b0, p0, p_out):
    """Dense torch form of eq. (14) with a carried state A_0 = a0 e^p0, B_0 = b0 e^p0:
    y_t = (eps^t A_0 + sum_{i<t} ...) / (eps^t B_0 + sum_{i<t} ... + e^{u+k_t}), and the state
    after the last token in units of e^{p_out}."""
    import torch
    B, T, C = k.shape
    t = torch.arange(T, dtype=torch.float64)
    dist = (t[:, None] - 1.0 - t[None, :])
    mask = (t[None, :] < t[:, None])
    kk, vv = k.permute(0, 2, 1), v.permute(0, 2, 1)
    expo = -dist[None, None] * w[None, :, None, None] + kk[:, :, None, :]
    E = torch.exp(torch.where(mask[None, None], expo, torch.full_like(expo, -torch.inf)))
    cur = torch.exp(u[None, :, None] + kk)
    decay = torch.exp(-t[None, None, :] * w[None, :, None])  # eps^t
    A0 = (a0 * torch.exp(p0)).unsqueeze(-1)
    B0 = (b0 * torch.exp(p0)).unsqueeze(-1)
    y = ((E * vv[:, :, None, :]).sum(-1) + decay * A0 + cur * vv) / (E.sum(-1) + decay * B0 + cur)
    wT = torch.exp(-(T - 1.0 - t)[None, None, :] * w[None, :, None] + kk)  # eps^{T-1-i} e^{k_i}
    AT = (wT * vv).sum(-1) + torch.exp(-T * w)[None, :] * A0[..., 0]
    BT = wT.sum(-1) + torch.exp(-T * w)[None, :] * B0[..., 0]
    return y.permute(0, 2, 1), AT * torch.exp(-p_out), BT * torch.exp(-p_out)


def mingru_torch(kz, h, x0=None):
    """minGRU as a plain torch loop: z = sigmoid(kz), x_t = (1 - z_t) x_{t-1} + z_t h_t."""
    import torch
    z = torch.sigmoid(kz)
    return scan_torch(1.0 - z, z * h, x0)


def minlstm_torch(kf, ki, h, x0=None):
    """minLSTM as a plain torch loop: f, i = sigmoid(kf), sigmoid(ki),
    x_t = f/(f+i) x_{t-1} + i/(f+i) h_t."""
    import torch
    f, i = torch.sigmoid(kf), torch.sigmoid(ki)
    return scan_torch(f / (f + i), i / (f + i) * h, x0)


def lru_normalized_torch(lam, u, x0=None):
    """x_t = lam x_{t-1} + sqrt(1 - |lam|^2) u_t as a plain torch loop (complex)."""
    import torch
    gamma = torch.sqrt(1.0 - lam.abs() ** 2)
    return scan_torch(lam, gamma * u, x0)


def wkv4_cond_sums(w, u, k, v, gy, r=None, s_in=None, gs_out=None):
    """(gw, gu, cw, cu, s_out) of WKV-4 (RWKV-LLM page, eq. (14), its chain rule; the gate of
    eq. (15); a carried state (a, b, p) decayed with the sums), every sum over the earlier
    steps written out: dL/dw, dL/du, and per channel the sums of the magnitudes of the
    products in their terms (cw with |A'| = A' over |v_i|).  s_out is (A_T, B_T, 0), the
    state after the last token at exponent 0.  No rescaling: for tiny inputs only."""
    B, T, C = k.shape
    f = lambda x: np.asarray(x, dtype=np.float64)  # noqa: E731
    w, u, k, v, gy = f(w), f(u), f(k), f(v), f(gy)
    gw, gu, cw, cu = np.zeros(C), np.zeros(C), np.zeros(C), np.zeros(C)
    s_out = np.zeros((B, C, 3))
    for b in range(B):
        for c in range(C):
            eps = np.exp(-w[c])
            a0, b0, p0 = (f(s_in[b, c]) if s_in is not None else (0.0, 0.0, 0.0))
            for t in range(T + 1):
                i = np.arange(t)
                e = eps ** (t - 1 - i) * np.exp(k[b, i, c])
                d = (t - 1 - i).astype(np.float64)
                st = eps ** t * np.exp(p0)  # the carried state, decayed to step t
                A = np.sum(e * v[b, i, c]) + st * a0
                Bs = np.sum(e) + st * b0
                Ad = np.sum(d * e * v[b, i, c]) + t * st * a0
                Adabs = np.sum(d * e * np.abs(v[b, i, c])) + t * st * abs(a0)
                Bd = np.sum(d * e) + t * st * b0
                if t == T:
                    s_out[b, c] = (A, Bs, 0.0)
                    if gs_out is not None:
                        gA, gB = f(gs_out[b, c])
                        gw[c] -= gA * Ad + gB * Bd
                        cw[c] += abs(gA) * Adabs + abs(gB) * Bd
                    break
                beta = np.exp(u[c] + k[b, t, c])
                D = Bs + beta
                y = (A + beta * v[b, t, c]) / D
                g = gy[b, t, c] * (1.0 / (1.0 + np.exp(-f(r[b, t, c]))) if r is not None else 1.0)
                gu[c] += g * beta * (v[b, t, c] - y) / D
                gw[c] -= g * (Ad - y * Bd) / D
                cu[c] += abs(g) * beta * (abs(v[b, t, c]) + abs(y)) / D
                cw[c] += abs(g) * (Adabs + abs(y) * Bd) / D
    return gw, gu, cw, cu, s_out
