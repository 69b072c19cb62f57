"""Host-side checks of the input generators and of the oracle's thread independence."""

import os
import subprocess
import sys

import numpy as np

from linear_recurrence_rnn_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_blockwise_draws_equal_one_draw(monkeypatch):
    # Drawing a large tensor in blocks gives the same stream as one draw.
    monkeypatch.setattr(workloads, "_BLOCK", 7)
    small = workloads.make_inputs(3, shape=(2, 9, 5))
    monkeypatch.setattr(workloads, "_BLOCK", 1 << 24)
    big = workloads.make_inputs(3, shape=(2, 9, 5))
    for key in small:
        np.testing.assert_array_equal(small[key], big[key])
    rng = np.random.default_rng(1003)
    w = np.exp(rng.uniform(-3, 1, 5)).astype(np.float32)
    u = (rng.standard_normal(5) * 0.5).astype(np.float32)
    k = (rng.standard_normal((2, 9, 5)) * 2.0).astype(np.float32)
    np.testing.assert_array_equal(big["w"], w)
    np.testing.assert_array_equal(big["u"], u)
    np.testing.assert_array_equal(big["k"], k)
    monkeypatch.setattr(workloads, "_BLOCK", 5)
    a = workloads.make_inputs(5, shape=(1, 6, 4))
    monkeypatch.setattr(workloads, "_BLOCK", 1 << 24)
    b = workloads.make_inputs(5, shape=(1, 6, 4))
    np.testing.assert_array_equal(a["u"], b["u"])
    monkeypatch.setattr(workloads, "_BLOCK", 3)
    a = workloads.make_inputs(4, shape=(2, 5, 3))
    monkeypatch.setattr(workloads, "_BLOCK", 1 << 24)
    b = workloads.make_inputs(4, shape=(2, 5, 3))
    np.testing.assert_array_equal(a["a"], b["a"])
    np.testing.assert_array_equal(a["b"], b["b"])


def test_distributions():
    d = workloads.make_inputs(2)
    assert d["k"].dtype == np.float32 and d["k"].shape == (8, 1024, 768)
    assert np.all(d["w"] > 0) and np.all(d["w"] >= np.exp(-3.0) * 0.999)
    assert np.all(d["w"] <= np.exp(1.0) * 1.001)
    assert abs(float(np.std(d["k"])) - 1.0) < 0.01
    assert abs(float(np.std(d["u"])) - 0.5) < 0.05
    d = workloads.make_inputs(5, shape=(1, 4096, 64))
    r = np.abs(d["lam"])
    th = np.angle(d["lam"])
    assert np.all((r >= 0.9 - 1e-6) & (r < 0.999 + 1e-6))
    assert np.all((th >= -1e-7) & (th < np.pi / 10 + 1e-6))
    assert abs(float(np.mean(np.abs(d["u"]) ** 2)) - 1.0) < 0.02
    d = workloads.make_inputs(4, shape=(4, 256, 32))
    assert np.all((d["a"] > 0) & (d["a"] < 1))


def test_oracle_is_thread_count_independent(tmp_path):
    script = (
        "import sys, numpy as np; sys.path.insert(0, %r)\n"
        "import oracle\n"
        "from linear_recurrence_rnn_amd import workloads\n"
        "d = workloads.make_inputs(3, shape=(3, 200, 37))\n"
        "y = oracle.wkv4_forward(d['w'], d['u'], d['k'], d['v'])\n"
        "g = oracle.wkv4_backward(d['w'], d['u'], d['k'], d['v'], d['gy'])\n"
        "np.savez(sys.argv[1], y=y, gw=g[0], gu=g[1], gk=g[2], gv=g[3], n=oracle.num_threads())\n"
    ) % ROOT
    outs = []
    for nt in ("1", "5"):
        path = str(tmp_path / ("o%s.npz" % nt))
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        subprocess.run([sys.executable, "-c", script, path], check=True, env=env)
        outs.append(np.load(path))
    assert int(outs[0]["n"]) == 1 and int(outs[1]["n"]) == 5
    for key in ("y", "gw", "gu", "gk", "gv"):
        np.testing.assert_array_equal(outs[0][key], outs[1][key])
