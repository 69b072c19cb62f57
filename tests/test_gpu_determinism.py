"""Results of the look-back scans do not depend on timing, through the C ABI.

A slab's carry is the nearest published inclusive prefix folded with the aggregates after it,
in chain order; which records a slab finds depends on timing, so the fold must give the same
bits on every path (lookback.hpp).  Each call below runs six times, every other time while a
large elementwise kernel runs on another stream (default priority), and every run must equal
the first bit for bit: the WKV-4 forward (eq. (14) of the RWKV-LLM page, "Time-mixing block"),
the checkpointing forward and the backward from its kept sums, the plain backward (its state
kernel's chain of forward sums), and the real scan (the minGRU page's recurrence).  Shapes
have tens of slabs per sequence, so the look-backs have many paths to take.
"""

import sys

import numpy as np
import pytest

from linear_recurrence_rnn_amd import workloads

pytestmark = pytest.mark.gpu

RUNS = 6


def announce(msg):
    sys.__stderr__.write("[gpu case] %s\n" % msg)
    sys.__stderr__.flush()


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401
    from linear_recurrence_rnn_amd import binding
    binding.load()
    return binding


def repeat(fn):
    """fn()'s host outputs for RUNS runs, odd runs beside a concurrent kernel on a side stream."""
    import torch
    noise_in = torch.ones(1 << 28, device="cuda")
    noise_out = torch.empty_like(noise_in)
    side = torch.cuda.Stream()
    runs = []
    for i in range(RUNS):
        torch.cuda.synchronize()
        if i % 2:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                torch.mul(noise_in, 1.5, out=noise_out)
        outs = fn()
        torch.cuda.synchronize()
        runs.append([t.cpu().numpy().copy() for t in outs])
    return runs


def check_same(runs, what):
    for i, r in enumerate(runs[1:], 1):
        for j, (a, b) in enumerate(zip(runs[0], r)):
            assert np.array_equal(a, b), (what, "run", i, "output", j)


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def kept_entries(ck, B, T, C):
    """The written entries of a checkpoint buffer: records of 5 dwords per lane per kept-sum
    position (every 56 steps strictly inside the sequence) and channel group of 64; lanes
    past the last channel and the position at or past T are never written."""
    ngrp, nck = (C + 63) // 64, (T + 55) // 56
    r = ck.view(np.uint32).reshape(B, ngrp, nck, 5, 64)[:, :, :(T - 1) // 56]
    return np.concatenate([r[:, g, ..., :min(64, C - 64 * g)].ravel() for g in range(ngrp)])


def test_wkv_forward_and_ckpt_step_bits_independent_of_timing(L):
    B, T, C = 4, 6000, 200  # 47 forward slabs of 128, 108 kept sums every 56
    announce("wkv4 forward / checkpointed step, %d runs, B=%d T=%d C=%d" % (RUNS, B, T, C))
    d = workloads.make_inputs(3, seed=71, shape=(B, T, C))
    w, u, k, v, gy = (dev(d[n]) for n in ("w", "u", "k", "v", "gy"))
    check_same(repeat(lambda: [L.wkv4_forward(w, u, k, v)]), "wkv4_forward")

    def step():
        y, ck = L.wkv4_forward_ckpt(w, u, k, v)
        return [y, ck] + list(L.wkv4_backward_ckpt(w, u, k, v, gy, ck))
    runs = repeat(step)
    for r in runs:
        r[1] = kept_entries(r[1], B, T, C)
    check_same(runs, "checkpointed step")


def test_wkv_forward_short_chain_bits_independent_of_timing(L):
    # The bench shape: chains of 8 slabs, which publish aggregates only and fold all of them.
    B, T, C = 8, 1024, 768
    announce("wkv4 forward (short chains), %d runs, B=%d T=%d C=%d" % (RUNS, B, T, C))
    d = workloads.make_inputs(2, seed=73, shape=(B, T, C))
    w, u, k, v = (dev(d[n]) for n in ("w", "u", "k", "v"))
    check_same(repeat(lambda: [L.wkv4_forward(w, u, k, v)]), "wkv4_forward")


def test_wkv_backward_bits_independent_of_timing(L):
    B, T, C = 4, 6000, 200  # 108 slabs of 56 steps; the state kernel's chain over them
    announce("wkv4_backward, %d runs, B=%d T=%d C=%d" % (RUNS, B, T, C))
    d = workloads.make_inputs(3, seed=72, shape=(B, T, C))
    w, u, k, v, gy = (dev(d[n]) for n in ("w", "u", "k", "v", "gy"))
    check_same(repeat(lambda: list(L.wkv4_backward(w, u, k, v, gy))), "wkv4_backward")


def test_real_scan_bits_independent_of_timing(L):
    B, T, C = 4, 20000, 256
    announce("linrec_scan_real, %d runs, B=%d T=%d C=%d" % (RUNS, B, T, C))
    m = workloads.make_mingru(B, T, C, seed=73)
    a, b = dev(m["a"]), dev(m["b"])
    check_same(repeat(lambda: [L.scan_real(a, b)]), "scan_real")
