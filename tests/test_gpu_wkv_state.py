"""GPU parity of wkv4_forward_ex (carried state and receptance gate, RWKV-LLM page,
"Time-mixing block", eqs. (14)-(15)) against the fp64 oracle, through the C ABI.

States are compared through what they determine: the ratio A/B = a/b and log B =
p + log b (the library picks its own scale p).  Tolerance: 1e-4 relative (RMS-floored
for y), as for the plain forward.
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


def random_state(B, C, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.standard_normal((B, C)), rng.uniform(0.2, 3.0, (B, C)), rng.uniform(-5, 20, (B, C))],
                    axis=-1).astype(np.float32)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("shape", [(8, 1024, 768), (3, 333, 100), (2, 1, 64)], ids=str)
def test_state_and_gate(L, shape, gated):
    announce("wkv4_forward_ex %s gated=%s" % (shape, gated))
    B, T, C = shape
    d = workloads.make_inputs(2, seed=40, shape=shape)
    r = np.random.default_rng(41).standard_normal(shape).astype(np.float32) * 2 if gated else None
    s_in = random_state(B, C, 42)
    y, s_out = L.wkv4_forward_ex(dev(d["w"]), dev(d["u"]), dev(d["k"]), dev(d["v"]), r=dev(r), state=dev(s_in))
    ry, rs = oracle.wkv4_forward_ex(d["w"], d["u"], d["k"], d["v"], r=r, s_in=s_in)
    assert rel_err(host(y), ry) <= TOL
    assert state_err(host(s_out), rs) <= TOL


def test_plain_call_is_wkv4_forward(L):
    announce("wkv4_forward_ex without state or gate == wkv4_forward B=2 T=700 C=96")
    d = workloads.make_inputs(3, seed=43, shape=(2, 700, 96))
    args = [dev(d[n]) for n in ("w", "u", "k", "v")]
    y1, _ = L.wkv4_forward_ex(*args, want_state=False)
    y2 = L.wkv4_forward(*args)
    np.testing.assert_array_equal(host(y1), host(y2))


@pytest.mark.parametrize("split", [1, 128, 500, 999])
def test_state_chains_calls(L, split):
    announce("wkv4_forward_ex split at %d of B=2 T=1000 C=130" % split)
    d = workloads.make_inputs(3, seed=44, shape=(2, 1000, 130))
    ref = oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])
    w, u = dev(d["w"]), dev(d["u"])
    y1, s = L.wkv4_forward_ex(w, u, dev(d["k"][:, :split]), dev(d["v"][:, :split]))
    y2, _ = L.wkv4_forward_ex(w, u, dev(d["k"][:, split:]), dev(d["v"][:, split:]), state=s)
    assert rel_err(np.concatenate([host(y1), host(y2)], axis=1), ref) <= TOL


def test_decode_token_by_token(L):
    announce("wkv4_forward_ex decode T=1 x 64 steps B=4 C=256")
    d = workloads.make_inputs(2, seed=45, shape=(4, 64, 256))
    ref = oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])
    w, u = dev(d["w"]), dev(d["u"])
    s = None
    ys = []
    for t in range(64):
        y, s = L.wkv4_forward_ex(w, u, dev(d["k"][:, t:t + 1]), dev(d["v"][:, t:t + 1]), state=s)
        ys.append(host(y))
    assert rel_err(np.concatenate(ys, axis=1), ref) <= TOL


def test_no_tokens_passes_state_through(L):
    import torch
    announce("wkv4_forward_ex T=0 state pass-through")
    B, C = 3, 70
    s_in = random_state(B, C, 46)
    e = torch.empty((B, 0, C), device="cuda")
    w = torch.ones(C, device="cuda")
    _, s_out = L.wkv4_forward_ex(w, w, e, e, state=dev(s_in))
    np.testing.assert_array_equal(host(s_out), s_in)
    _, s_out = L.wkv4_forward_ex(w, w, e, e)
    np.testing.assert_array_equal(host(s_out), 0.0)
