"""GPU parity of wkv4_decode_step (one token of WKV-4 in recurrent form, RWKV-LLM page,
"Time-mixing block" eqs. (14)-(15) and "并行训练和序列解码") against the fp64 oracle,
through the C ABI.

One step is the oracle's forward with a carried state over a single token; T steps are the
oracle's forward over all T tokens.  States are compared through what they determine (A/B
and log B), as in the state tests of the chunked forward.  Tolerance: 1e-4 relative
(RMS-floored for y): each step rounds the state to float32 once (relative 6e-8), so a few
hundred steps stay two orders of magnitude inside it.
"""

import sys

import numpy as np
import pytest

import oracle
from oracle.compare import rel_err
from linear_recurrence_rnn_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4


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


def state_err(got, ref):
    """Largest relative error of A/B and of log B between two (a, b, p) states."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ratio_g, ratio_r = got[..., 0] / got[..., 1], ref[..., 0] / ref[..., 1]
    logb_g, logb_r = got[..., 2] + np.log(got[..., 1]), ref[..., 2] + np.log(ref[..., 1])
    e1 = np.max(np.abs(ratio_g - ratio_r) / np.maximum(np.abs(ratio_r), np.sqrt(np.mean(ratio_r ** 2))))
    e2 = np.max(np.abs(logb_g - logb_r) / np.maximum(np.abs(logb_r), 1.0))
    return max(e1, e2)


def random_state(B, C, seed, p_lo=-5.0, p_hi=20.0):
    rng = np.random.default_rng(seed)
    return np.stack([rng.standard_normal((B, C)), rng.uniform(0.2, 3.0, (B, C)), rng.uniform(p_lo, p_hi, (B, C))],
                    axis=-1).astype(np.float32)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("start", ["empty", "random"])
@pytest.mark.parametrize("shape", [(8, 768), (3, 100), (1, 1)], ids=str)
def test_one_step(L, shape, start, gated):
    announce("wkv4_decode_step %s start=%s gated=%s" % (shape, start, gated))
    B, C = shape
    d = workloads.make_inputs(2, seed=50, shape=(B, 1, C))
    r = np.random.default_rng(51).standard_normal((B, 1, C)).astype(np.float32) * 2 if gated else None
    s_in = random_state(B, C, 52) if start == "random" else np.zeros((B, C, 3), np.float32)
    st = dev(s_in)
    y = L.wkv4_decode_step(dev(d["w"]), dev(d["u"]), dev(d["k"][:, 0]), dev(d["v"][:, 0]), st,
                           r=None if r is None else dev(r[:, 0]))
    ry, rs = oracle.wkv4_forward_ex(d["w"], d["u"], d["k"], d["v"], r=r, s_in=s_in)
    assert rel_err(host(y), ry[:, 0]) <= TOL
    assert state_err(host(st), rs) <= TOL


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("wid,shape", [(2, (4, 200, 96)), (3, (2, 300, 130))], ids=str)
def test_steps_follow_the_forward(L, wid, shape, gated):
    announce("wkv4_decode_step x T vs oracle forward wid=%d %s gated=%s" % (wid, shape, gated))
    import torch
    B, T, C = shape
    d = workloads.make_inputs(wid, seed=53, shape=shape)
    r = np.random.default_rng(54).standard_normal(shape).astype(np.float32) if gated else None
    w, u = dev(d["w"]), dev(d["u"])
    k, v = dev(d["k"]), dev(d["v"])
    rr = dev(r)
    st = torch.zeros((B, C, 3), dtype=torch.float32, device="cuda")
    ys = []
    for t in range(T):
        ys.append(L.wkv4_decode_step(w, u, k[:, t].contiguous(), v[:, t].contiguous(), st,
                                     r=None if rr is None else rr[:, t].contiguous()))
    y = torch.stack(ys, dim=1)
    ry, rs = oracle.wkv4_forward_ex(d["w"], d["u"], d["k"], d["v"], r=r)
    assert rel_err(host(y), ry) <= TOL
    assert state_err(host(st), rs) <= TOL


def test_decode_continues_the_chunked_forward(L):
    """Prefill with wkv4_forward_ex, then decode: together they are one forward."""
    announce("wkv4_forward_ex prefill 900 + 40 decode steps B=3 C=200")
    import torch
    B, T, C, T0 = 3, 940, 200, 900
    d = workloads.make_inputs(2, seed=55, shape=(B, T, C))
    r = np.random.default_rng(56).standard_normal((B, T, C)).astype(np.float32)
    w, u = dev(d["w"]), dev(d["u"])
    k, v, rr = dev(d["k"]), dev(d["v"]), dev(r)
    y0, st = L.wkv4_forward_ex(w, u, k[:, :T0].contiguous(), v[:, :T0].contiguous(), r=rr[:, :T0].contiguous())
    ys = [y0]
    for t in range(T0, T):
        ys.append(L.wkv4_decode_step(w, u, k[:, t].contiguous(), v[:, t].contiguous(), st,
                                     r=rr[:, t].contiguous())[:, None])
    y = torch.cat(ys, dim=1)
    ry, rs = oracle.wkv4_forward_ex(d["w"], d["u"], d["k"], d["v"], r=r)
    assert rel_err(host(y), ry) <= TOL
    assert state_err(host(st), rs) <= TOL


def test_extreme_exponents(L):
    """k spikes of +-60 and states at e^{+-80}: the integer base-2 exponents keep every step
    finite where e^{k} and e^{p} alone would overflow or underflow float32."""
    announce("wkv4_decode_step extreme exponents B=4 C=64 T=50")
    import torch
    B, T, C = 4, 50, 64
    rng = np.random.default_rng(57)
    d = workloads.make_inputs(2, seed=58, shape=(B, T, C))
    k = d["k"].copy()
    spikes = rng.random((B, T, C)) < 0.1
    k[spikes] = rng.choice([-60.0, 60.0], size=int(spikes.sum())).astype(np.float32)
    s_in = random_state(B, C, 59, p_lo=-80.0, p_hi=80.0)
    w, u, kd, vd = dev(d["w"]), dev(d["u"]), dev(k), dev(d["v"])
    st = dev(s_in)
    ys = [L.wkv4_decode_step(w, u, kd[:, t].contiguous(), vd[:, t].contiguous(), st) for t in range(T)]
    y = host(torch.stack(ys, dim=1))
    ry, rs = oracle.wkv4_forward_ex(d["w"], d["u"], k, d["v"], s_in=s_in)
    assert np.all(np.isfinite(y))
    assert rel_err(y, ry) <= TOL
    assert state_err(host(st), rs) <= TOL


def test_empty_batch_is_a_no_op(L):
    import torch
    z = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    st = torch.zeros((0, 8, 3), dtype=torch.float32, device="cuda")
    w = torch.zeros(8, dtype=torch.float32, device="cuda")
    y = L.wkv4_decode_step(w, w, z, z, st)
    assert tuple(y.shape) == (0, 8)
