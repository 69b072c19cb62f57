"""GPU parity of rwkv_token_shift and its backward (RWKV-LLM page, "Time-mixing block", eqs.
(11)-(13)) against the fp64 oracle, through the C ABI.

Tolerance 1e-6 relative, floored at the RMS of the whole output: each output is one fused
multiply-add of float32 inputs (forward), or a short sum (gx), so its error is a few float32
ulps of the operands' scale.  An interpolation can cancel to ~0 at any element, and a short
sequence gives no per-sequence floor (T = 1), hence the whole-tensor floor.  gmu is a
float64 sum of B*T products, compared at 1e-6 of its RMS over channels.
"""

import sys

import numpy as np
import pytest

import oracle
from oracle.compare import rel_err
from linear_recurrence_rnn_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-6


def announce(msg):
    sys.__stderr__.write("[gpu case] %s\n" % msg)
    sys.__stderr__.flush()


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401
    from linear_recurrence_rnn_amd import binding
    binding.load()
    return binding


def dev(x):
    import torch
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return None if t is None else t.cpu().numpy()


SHAPES = [(8, 1024, 768, 3), (3, 333, 100, 3), (2, 17, 7, 2), (1, 1, 64, 1), (4, 130, 258, 4)]


@pytest.mark.parametrize("with_prev", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_forward(L, shape, with_prev):
    B, T, C, M = shape
    announce("rwkv_token_shift %s prev=%s" % (shape, with_prev))
    d = workloads.make_token_shift(B, T, C, M, 60)
    xp = d["x_prev"] if with_prev else None
    got = host(L.token_shift(dev(d["x"]), dev(d["mu"]), dev(xp)))
    ref = oracle.token_shift(d["x"], d["mu"], xp)
    for m in range(M):
        assert rel_err(got[m], ref[m], None) <= TOL, m


@pytest.mark.parametrize("with_prev", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_backward(L, shape, with_prev):
    B, T, C, M = shape
    announce("rwkv_token_shift_backward %s prev=%s" % (shape, with_prev))
    d = workloads.make_token_shift(B, T, C, M, 61, with_grad=True)
    xp = d["x_prev"] if with_prev else None
    gx, gmu, gxp = (host(t) for t in L.token_shift_backward(dev(d["x"]), dev(d["mu"]), dev(d["g"]), dev(xp),
                                                               want_gx_prev=True))
    rgx, rgmu, rgxp = oracle.token_shift_backward(d["x"], d["mu"], d["g"], xp)
    assert rel_err(gx, rgx, None) <= TOL
    assert rel_err(gmu, rgmu, None) <= TOL
    assert rel_err(gxp[:, None, :], rgxp[:, None, :], None) <= TOL


@pytest.mark.parametrize("vec", ["1", "2"])
def test_narrow_lanes(L, vec, monkeypatch):
    """Forced 1 or 2 channels per lane give the same results (other kernel instances)."""
    monkeypatch.setenv("LINREC_VEC", vec)
    B, T, C, M = 3, 100, 96, 3
    announce("token shift LINREC_VEC=%s" % vec)
    d = workloads.make_token_shift(B, T, C, M, 62, with_grad=True)
    got = host(L.token_shift(dev(d["x"]), dev(d["mu"]), dev(d["x_prev"])))
    ref = oracle.token_shift(d["x"], d["mu"], d["x_prev"])
    assert max(rel_err(got[m], ref[m], None) for m in range(M)) <= TOL
    gx, gmu, gxp = (host(t) for t in L.token_shift_backward(dev(d["x"]), dev(d["mu"]), dev(d["g"]), dev(d["x_prev"])))
    rgx, rgmu, rgxp = oracle.token_shift_backward(d["x"], d["mu"], d["g"], d["x_prev"])
    assert rel_err(gx, rgx, None) <= TOL and rel_err(gmu, rgmu, None) <= TOL


def test_chained_calls_equal_one(L):
    """Two calls chained through x_prev give the outputs of one call over the whole sequence."""
    import torch
    B, T, C, M = 2, 200, 64, 3
    announce("token shift chained 120 + 80")
    d = workloads.make_token_shift(B, T, C, M, 63)
    x = dev(d["x"])
    whole = host(L.token_shift(x, dev(d["mu"])))
    a = L.token_shift(x[:, :120].contiguous(), dev(d["mu"]))
    b = L.token_shift(x[:, 120:].contiguous(), dev(d["mu"]), x[:, 119].contiguous())
    assert np.array_equal(host(torch.cat([a, b], dim=2)), whole)


def test_gmu_is_deterministic(L):
    B, T, C, M = 4, 777, 192, 3
    announce("token shift backward determinism")
    d = workloads.make_token_shift(B, T, C, M, 64, with_grad=True)
    args = (dev(d["x"]), dev(d["mu"]), dev(d["g"]), dev(d["x_prev"]))
    r1 = [host(t) for t in L.token_shift_backward(*args)]
    r2 = [host(t) for t in L.token_shift_backward(*args)]
    for u, v in zip(r1, r2):
        assert np.array_equal(u, v)


def test_empty_sequence_zero_fills(L):
    import torch
    announce("token shift backward T=0")
    x = torch.zeros((2, 0, 8), dtype=torch.float32, device="cuda")
    mu = torch.ones((3, 8), dtype=torch.float32, device="cuda")
    g = torch.zeros((3, 2, 0, 8), dtype=torch.float32, device="cuda")
    gmu0 = torch.full((3, 8), 7.0, device="cuda")
    gxp0 = torch.full((2, 8), 7.0, device="cuda")
    gx, gmu, gxp = L.token_shift_backward(x, mu, g, torch.zeros((2, 8), device="cuda"),
                                          out=(torch.empty_like(x), gmu0, gxp0))
    assert np.all(host(gmu) == 0) and np.all(host(gxp) == 0)
