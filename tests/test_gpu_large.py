"""Parity beyond 4 GiB per tensor, through the C ABI: every (B,T,C) operand here holds more
than 2^32 bytes, so row offsets past 32 bits are exercised (each slab's rows are addressed
from a 64-bit base).  Shapes: B=1, C=1000 (the last channel group is partial), T of about a
million steps (the last slab is partial).

Inputs are drawn on the GPU with a seeded torch generator (the host generators would take
minutes at this size): k, v, gy ~ N(0, 1), the WKV channel parameters as the workloads draw
them; the real scan's a ~ U(0, 1), b ~ N(0, 1); the complex scan's u ~ complex N(0, 1) and
lambda = r e^{i theta}, r ~ U(0.9, 0.999), theta ~ U(0, pi/10) (the LRU workload's ranges).
The outputs are compared with the fp64 oracle on sampled channels, whole sequences each,
including both ends of the partial group: eq. (14) of the RWKV-LLM page ("Time-mixing block")
and its chain rule, the real scan of the minGRU page, the complex diagonal recurrence of the
LRU write-up.  Tolerances as in the other parity tests: 1e-4 (float32), 1e-3 for the complex
scan over 6e5 steps (as for the LRU workload at T = 262144); dL/dw and dL/du channel by
channel against their conditioning sums.
"""

import math
import sys

import numpy as np
import pytest

import oracle
from oracle.compare import chan_ratio, rel_err
from linear_recurrence_rnn_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4
C = 1000
CS = [0, 1, 517, 959, 960, 999]  # sampled channels; 960 .. 999 form the partial last group


def announce(msg):
    sys.__stderr__.write("[gpu case] %s\n" % msg)
    sys.__stderr__.flush()


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401
    from linear_recurrence_rnn_amd import binding
    binding.load()
    return binding


def gen(seed):
    import torch
    return torch.Generator(device="cuda").manual_seed(seed)


def sample(t):
    """The sampled channels of a (1,T,C) device tensor, on the host."""
    import torch
    idx = torch.tensor(CS, device=t.device)
    return t.index_select(2, idx).cpu().numpy()


@pytest.fixture(autouse=True)
def release_memory():
    """Hands the cached device memory back after each test (tens of GiB here)."""
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_wkv_forward_backward_beyond_4gib(L):
    import torch
    T = 1_100_000
    assert T * C * 4 > 2 ** 32
    announce("wkv4_forward / wkv4_backward B=1 T=%d C=%d (%.1f GiB per tensor)" % (T, C, T * C * 4 / 2 ** 30))
    w_h, u_h = workloads.wkv_params(np.random.default_rng(901), C)
    w, u = torch.from_numpy(w_h).cuda(), torch.from_numpy(u_h).cuda()
    g = gen(902)
    k = torch.randn((1, T, C), generator=g, device="cuda")
    v = torch.randn((1, T, C), generator=g, device="cuda")
    y = L.wkv4_forward(w, u, k, v)
    ks, vs = sample(k), sample(v)
    ref = oracle.wkv4_forward(w_h[CS], u_h[CS], ks, vs)
    err = rel_err(sample(y), ref)
    assert err <= TOL, err
    del y
    gy = torch.randn((1, T, C), generator=g, device="cuda")
    gw, gu, gk, gv = L.wkv4_backward(w, u, k, v, gy)
    full = oracle.wkv4_backward_cond(w_h[CS], u_h[CS], ks, vs, sample(gy))
    errs = {"gk": rel_err(sample(gk), full[2]), "gv": rel_err(sample(gv), full[3]),
            "gw": chan_ratio(gw.cpu().numpy()[CS], full[0], full[6], TOL) * TOL,
            "gu": chan_ratio(gu.cpu().numpy()[CS], full[1], full[7], TOL) * TOL}
    assert all(e <= TOL for e in errs.values()), errs


def test_scan_real_beyond_4gib(L):
    import torch
    T = 1_100_000
    announce("linrec_scan_real B=1 T=%d C=%d" % (T, C))
    g = gen(903)
    a = torch.rand((1, T, C), generator=g, device="cuda")
    b = torch.randn((1, T, C), generator=g, device="cuda")
    x = L.scan_real(a, b)
    ref = oracle.scan_real(sample(a), sample(b))
    err = rel_err(sample(x), ref)
    assert err <= TOL, err


def test_scan_complex_beyond_4gib(L):
    import torch
    T = 600_000
    assert T * C * 8 > 2 ** 32
    announce("linrec_scan_complex B=1 T=%d C=%d" % (T, C))
    rng = np.random.default_rng(904)
    lam_h = (rng.uniform(0.9, 0.999, C) * np.exp(1j * rng.uniform(0.0, math.pi / 10, C))).astype(np.complex64)
    g = gen(905)
    u = torch.complex(torch.randn((1, T, C), generator=g, device="cuda"),
                      torch.randn((1, T, C), generator=g, device="cuda"))
    x = L.scan_complex(torch.from_numpy(lam_h).cuda(), u)
    ref = oracle.scan_complex(lam_h[CS], sample(u))
    err = rel_err(sample(x), ref)
    assert err <= 1e-3, err
