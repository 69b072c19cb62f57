"""GPU parity of wkv4_backward_ex: the backward of the gated time-mix output
o = sigma(r) wkv (RWKV-LLM page, "Time-mixing block", eq. (15)) against the fp64 oracle,
through the C ABI.  Tolerance 1e-4 (RMS-floored; dL/dw and dL/du over channels), as for the
plain backward.
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
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(L, d, r):
    got = [host(t) for t in L.wkv4_backward_gated(dev(d["w"]), dev(d["u"]), dev(d["k"]), dev(d["v"]), dev(r),
                                                  dev(d["gy"]))]
    ref = oracle.wkv4_backward_gated(d["w"], d["u"], d["k"], d["v"], r, d["gy"])
    errs = {"gw": rel_err(got[0], ref[0], None), "gu": rel_err(got[1], ref[1], None),
            "gk": rel_err(got[2], ref[2]), "gv": rel_err(got[3], ref[3]), "gr": rel_err(got[4], ref[4])}
    if d["k"].shape[1] == 1:
        # One step: y_0 = v_0 exactly, so dL/dw, dL/du and dL/dk are 0; the oracle's values
        # are its own rounding noise (~1e-17), so compare absolutely.
        for name, i in (("gw", 0), ("gu", 1), ("gk", 2)):
            errs[name] = float(np.max(np.abs(got[i] - ref[i])))
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, errs


@pytest.mark.parametrize("shape", [(2, 1000, 256), (3, 333, 100), (1, 1, 64), (4, 2048, 128), (1, 4000, 64)], ids=str)
def test_gated_backward(L, shape):
    announce("wkv4_backward_ex %s" % (shape,))
    d = workloads.make_inputs(3, seed=80, shape=shape)
    r = (np.random.default_rng(81).standard_normal(shape) * 2).astype(np.float32)
    check(L, d, r)


def test_gated_backward_saturated_gates(L):
    """|r| up to ~40: sigma(r) is 0 or 1 and sigma'(r) underflows; dL/dr stays finite."""
    announce("wkv4_backward_ex saturated gates")
    d = workloads.make_inputs(3, seed=82, shape=(2, 700, 96))
    r = (np.random.default_rng(83).standard_normal(d["k"].shape) * 15).astype(np.float32)
    check(L, d, r)


def test_gated_backward_exact_path(L, monkeypatch):
    monkeypatch.setenv("LINREC_WKV_EXACT", "1")
    announce("wkv4_backward_ex exact path")
    d = workloads.make_inputs(3, seed=84, shape=(2, 900, 128))
    r = np.random.default_rng(85).standard_normal(d["k"].shape).astype(np.float32)
    check(L, d, r)


def test_gated_backward_recompute_path(L, monkeypatch):
    monkeypatch.setenv("LINREC_SPIN", "0")
    announce("wkv4_backward_ex with LINREC_SPIN=0")
    d = workloads.make_inputs(3, seed=86, shape=(1, 1500, 64))
    r = np.random.default_rng(87).standard_normal(d["k"].shape).astype(np.float32)
    check(L, d, r)


def test_open_gate_equals_plain_backward(L):
    """r = 60: sigma = 1 in float32, so the gradients equal wkv4_backward's bit for bit and
    dL/dr is 0 (sigma(-60) underflows to 0 in float32... or to ~1e-26)."""
    announce("wkv4_backward_ex open gate vs wkv4_backward")
    d = workloads.make_inputs(3, seed=88, shape=(2, 600, 128))
    r = np.full(d["k"].shape, 60.0, np.float32)
    got = [host(t) for t in L.wkv4_backward_gated(dev(d["w"]), dev(d["u"]), dev(d["k"]), dev(d["v"]), dev(r),
                                                  dev(d["gy"]))]
    plain = [host(t) for t in L.wkv4_backward(dev(d["w"]), dev(d["u"]), dev(d["k"]), dev(d["v"]), dev(d["gy"]))]
    for a, b in zip(got[:4], plain):
        assert np.array_equal(a, b)
    assert np.max(np.abs(got[4])) < 1e-20


def test_backward_bits_do_not_depend_on_timing(L):
    """Three runs of a many-slab backward (2340 slabs per call): the slabs' carries come from
    the early or the blocking look-back as timing decides, and fold the same records in the
    same order either way, so every output is bit-identical."""
    announce("wkv4_backward / gated: 3 runs, B=8 T=4096 C=256, bitwise")
    d = workloads.make_inputs(3, seed=89, shape=(8, 4096, 256))
    r = np.random.default_rng(90).standard_normal(d["k"].shape).astype(np.float32)
    args = [dev(d[n]) for n in ("w", "u", "k", "v")]
    runs = [[host(t) for t in L.wkv4_backward(*args, dev(d["gy"]))] for _ in range(3)]
    runs_g = [[host(t) for t in L.wkv4_backward_gated(*args, dev(r), dev(d["gy"]))] for _ in range(3)]
    for rr in (runs, runs_g):
        for other in rr[1:]:
            for a, b in zip(rr[0], other):
                np.testing.assert_array_equal(a, b)
