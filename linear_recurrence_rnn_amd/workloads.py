"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests and the bench.

This module draws random numbers and nothing else: it holds none of the recurrence
arithmetic, imports neither the HIP binding nor the oracle, and both sides receive
exactly the float32 / complex64 arrays produced here.

Workload shapes and distributions (``N(m, s)``: ``s`` is the standard deviation;
``U(a, b)`` is half-open):

==== ======================================== ================================================
id   workload                                 draws, in this order
==== ======================================== ================================================
1    WKV-4 forward, B=1 T=64 C=32             w=exp(U(-3,1)) (C); u~N(0,0.5) (C); k,v~N(0,1)
2    WKV-4 forward, B=8 T=1024 C=768          as 1
3    WKV-4 fwd+bwd, B=8 T=4096 C=2560         w, u as 1; k~N(0,2); v~N(0,1); gy~N(0,1)
4    minGRU scan, B=64 T=4096 C=256           z=sigmoid(N(0,1)); h~N(0,1); a=1-z, b=z*h; x0=0
5    LRU complex scan, B=1 T=262144 C=1024    r~U(0.9,0.999), theta~U(0,pi/10) (C);
                                              lam=r*exp(i*theta); u=(N(0,1)+i*N(0,1))/sqrt(2)
==== ======================================== ================================================

The per-channel decay ``w = exp(U(-3, 1))`` keeps ``w >= 0`` as the RWKV page requires for
its time-decay vector (RWKV-LLM page, "Transformers和AFT", eq. (10)); the minGRU gate
``a = 1 - z, b = z * h`` is the minGRU update written in the scan form
``v_t = a_t * v_{t-1} + b_t`` ("Were RNNs All We Needed?" news page, minGRU section); the
LRU eigenvalue ``lam = r * exp(i*theta)`` follows the LRU write-up's polar form (section on
the diagonal complex recurrence), with the ring and phase ranges of the workload table.

Every draw is made in float64 from ``numpy.random.default_rng(seed)`` (PCG64) and rounded
once to float32.  Large tensors are drawn in blocks from the same generator, which yields
the same stream as one large draw (checked in the CPU tests).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict

import numpy as np

_BLOCK = 1 << 24  # elements per fp64 block when drawing large tensors


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: which entry point it drives and its shape."""

    wid: int
    kind: str  # "wkv4_forward" | "wkv4_backward" | "scan_real" | "scan_complex"
    B: int
    T: int
    C: int
    seed: int
    label: str

    @property
    def elements(self) -> int:
        return self.B * self.T * self.C


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "wkv4_forward", 1, 64, 32, 1001, "WKV-4 forward fp32 B=1 T=64 C=32"),
    2: Workload(2, "wkv4_forward", 8, 1024, 768, 1002, "WKV-4 forward fp32 B=8 T=1024 C=768"),
    3: Workload(3, "wkv4_backward", 8, 4096, 2560, 1003,
                "WKV-4 forward+backward fp32 B=8 T=4096 C=2560, k~N(0,2)"),
    4: Workload(4, "scan_real", 64, 4096, 256, 1004, "minGRU real scan fp32 B=64 T=4096 C=256"),
    5: Workload(5, "scan_complex", 1, 262144, 1024, 1005,
                "LRU complex scan complex64 B=1 T=262144 C=1024"),
}


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """float64 N(0, scale) draws, rounded to float32, drawn in blocks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = rng.standard_normal(e - s) * scale
    return out.reshape(shape)


def _normal_into(rng: np.random.Generator, dst: np.ndarray, scale: float) -> None:
    """Fill the flat float32 view ``dst`` (may be strided) with N(0, scale) draws."""
    n = dst.shape[0]
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        dst[s:e] = rng.standard_normal(e - s) * scale


def wkv_params(rng: np.random.Generator, C: int):
    """Per-channel decay ``w = exp(U(-3, 1))`` (so ``w > 0``) and bonus ``u ~ N(0, 0.5)``."""
    w = np.exp(rng.uniform(-3.0, 1.0, size=C)).astype(np.float32)
    u = (rng.standard_normal(C) * 0.5).astype(np.float32)
    return w, u


def make_wkv(B: int, T: int, C: int, seed: int, k_std: float = 1.0, with_grad: bool = False):
    """WKV-4 inputs: w, u (C,), k, v (B,T,C) float32, and gy (B,T,C) if ``with_grad``."""
    rng = np.random.default_rng(seed)
    w, u = wkv_params(rng, C)
    k = _normal(rng, (B, T, C), k_std)
    v = _normal(rng, (B, T, C), 1.0)
    out = {"w": w, "u": u, "k": k, "v": v}
    if with_grad:
        out["gy"] = _normal(rng, (B, T, C), 1.0)
    return out


def make_mingru(B: int, T: int, C: int, seed: int):
    """minGRU scan inputs a = 1 - z, b = z * h (float64 then float32), x0 = None (zero).

    All of z is drawn first, then all of h, both blockwise from one generator.
    """
    rng = np.random.default_rng(seed)
    n = B * T * C
    z = np.empty(n, dtype=np.float64)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        z[s:e] = rng.standard_normal(e - s)
    z = 1.0 / (1.0 + np.exp(-z))  # sigmoid
    a = np.empty(n, dtype=np.float32)
    b = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        h = rng.standard_normal(e - s)
        a[s:e] = 1.0 - z[s:e]
        b[s:e] = z[s:e] * h
    return {"a": a.reshape(B, T, C), "b": b.reshape(B, T, C), "x0": None}


def make_lru(B: int, T: int, C: int, seed: int, r_lo: float = 0.9, r_hi: float = 0.999,
             theta_hi: float = math.pi / 10, with_x0: bool = False):
    """LRU scan inputs: lam (C,) complex64 with |lam| = r, arg lam = theta; u (B,T,C) complex64;
    with ``with_x0`` an initial state x0 (B,C) complex64 of the same distribution as u, drawn
    after u (else None)."""
    rng = np.random.default_rng(seed)
    r = rng.uniform(r_lo, r_hi, size=C)
    theta = rng.uniform(0.0, theta_hi, size=C)
    lam = (r * np.exp(1j * theta)).astype(np.complex64)
    u = np.empty((B, T, C), dtype=np.complex64)
    flat = u.reshape(-1).view(np.float32)
    s2 = 1.0 / math.sqrt(2.0)
    _normal_into(rng, flat[0::2], s2)
    _normal_into(rng, flat[1::2], s2)
    x0 = None
    if with_x0:
        x0 = np.empty((B, C), dtype=np.complex64)
        f0 = x0.reshape(-1).view(np.float32)
        _normal_into(rng, f0[0::2], s2)
        _normal_into(rng, f0[1::2], s2)
    return {"lam": lam, "u": u, "x0": x0}


def make_inputs(wid: int, seed: int | None = None, shape=None):
    """Inputs of workload ``wid`` (1..5); ``shape=(B,T,C)`` overrides the size only."""
    wl = WORKLOADS[wid]
    B, T, C = shape if shape is not None else (wl.B, wl.T, wl.C)
    seed = wl.seed if seed is None else seed
    if wid in (1, 2):
        return make_wkv(B, T, C, seed)
    if wid == 3:
        return make_wkv(B, T, C, seed, k_std=2.0, with_grad=True)
    if wid == 4:
        return make_mingru(B, T, C, seed)
    if wid == 5:
        return make_lru(B, T, C, seed)
    raise KeyError(wid)


def make_scan_adjoint_inputs(wid: int, host: dict, seed: int | None = None):
    """Extra inputs of a scan adjoint on workload ``wid`` (4: real, 5: complex) shaped like
    ``host``: the upstream gradient gx ~ N(0,1) (complex: (N(0,1) + i N(0,1))/sqrt 2) and a
    stand-in x of the same distribution for the forward output (for timing; parity tests
    take x from the oracle's forward scan)."""
    seed = (WORKLOADS[wid].seed if seed is None else seed) + 7919
    rng = np.random.default_rng(seed)
    if wid == 4:
        B, T, C = host["a"].shape
        return {"gx": _normal(rng, (B, T, C), 1.0), "x": _normal(rng, (B, T, C), 1.0)}
    if wid == 5:
        B, T, C = host["u"].shape
        out = {}
        for name in ("gx", "x"):
            z = np.empty((B, T, C), dtype=np.complex64)
            flat = z.reshape(-1).view(np.float32)
            _normal_into(rng, flat[0::2], 1.0 / math.sqrt(2.0))
            _normal_into(rng, flat[1::2], 1.0 / math.sqrt(2.0))
            out[name] = z
        return out
    raise KeyError(wid)


def make_token_shift(B: int, T: int, C: int, M: int, seed: int, with_grad: bool = False):
    """Token-shift inputs: x (B,T,C) ~ N(0,1), x_prev (B,C) ~ N(0,1), mu (M,C) ~ U(0,1), and
    g (M,B,T,C) ~ N(0,1) if ``with_grad``; all float32, drawn in that order."""
    rng = np.random.default_rng(seed)
    out = {"x": _normal(rng, (B, T, C), 1.0), "x_prev": _normal(rng, (B, C), 1.0),
           "mu": rng.uniform(0.0, 1.0, size=(M, C)).astype(np.float32)}
    if with_grad:
        out["g"] = _normal(rng, (M, B, T, C), 1.0)
    return out


def make_gated(B: int, T: int, C: int, seed: int, logit_std: float = 1.0, with_grad: bool = False):
    """Inputs of the gated scan variants: gate pre-activations kz, kf, ki ~ N(0, logit_std),
    candidates h ~ N(0,1), x0 ~ N(0,1) (B,C), a per-channel decay lam ~ U(-1, 1) (C,), and
    with ``with_grad`` an upstream gradient gx ~ N(0,1) (B,T,C); all float32, drawn in that
    order."""
    rng = np.random.default_rng(seed)
    out = {n: _normal(rng, (B, T, C), logit_std) for n in ("kz", "kf", "ki")}
    out["h"] = _normal(rng, (B, T, C), 1.0)
    out["x0"] = _normal(rng, (B, C), 1.0)
    out["lam"] = rng.uniform(-1.0, 1.0, size=C).astype(np.float32)
    if with_grad:
        out["gx"] = _normal(rng, (B, T, C), 1.0)
    return out
