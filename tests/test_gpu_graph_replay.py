"""Calls captured into a HIP graph and replayed, through the C ABI: every replay gives, bit
for bit, what an eager call on the replay's inputs gives, and stays within the oracle's
tolerance (WKV-4 forward, backward and the checkpointed training step: eq. (14) of the
RWKV-LLM page, "Time-mixing block"; the decay adjoint with its glambda sums: the LRU
write-up's diagonal recurrence).

A captured call keeps its host-drawn look-back tag on every replay; while the stream is
capturing, the library also records a fill kernel that clears the call's flags, so each
replay starts with none published.  Each replay here gets new inputs, and eager calls and
synchronisations run between replays.
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


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().copy()


def capture(fn):
    """Runs fn once eagerly on a side stream, then captures it; returns (graph, fn's
    outputs inside the graph)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def load(dst, arrays):
    import torch
    for t, a in zip(dst, arrays):
        t.copy_(torch.from_numpy(np.ascontiguousarray(a)))


# 12 slabs per row (the look-back runs, with inclusive prefixes); 8 slabs per row at the
# bench shape (a short chain: aggregates only)
@pytest.mark.parametrize("B,T,C", [(2, 1500, 200), (8, 1024, 768)], ids=["long_chain", "short_chain"])
def test_forward_graph_replays(L, B, T, C):
    import torch
    announce("wkv4_forward captured and replayed B=%d T=%d C=%d" % (B, T, C))
    d0 = workloads.make_inputs(1, seed=201, shape=(B, T, C))
    w, u, k, v = (torch.from_numpy(d0[n]).cuda() for n in ("w", "u", "k", "v"))
    y = torch.empty_like(k)
    ws = torch.empty(L.workspace_size("wkv4_forward", B, T, C), dtype=torch.uint8, device="cuda")
    g, _ = capture(lambda: L.wkv4_forward(w, u, k, v, out=y, workspace=ws))
    for seed in (202, 203, 204):
        d = workloads.make_inputs(1, seed=seed, shape=(B, T, C))
        load((w, u, k, v), (d["w"], d["u"], d["k"], d["v"]))
        g.replay()
        got = host(y)
        eager = host(L.wkv4_forward(w, u, k, v))
        assert np.array_equal(got, eager), seed
        assert rel_err(got, oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL, seed


def test_backward_graph_replays(L):
    import torch
    B, T, C = 2, 700, 130  # 13 slabs of 56 steps: both look-backs and the state kernel's chain
    announce("wkv4_backward captured and replayed B=%d T=%d C=%d" % (B, T, C))
    d0 = workloads.make_inputs(3, seed=205, shape=(B, T, C))
    ins = [torch.from_numpy(d0[n]).cuda() for n in ("w", "u", "k", "v", "gy")]
    outs = (torch.empty(C, device="cuda"), torch.empty(C, device="cuda"), torch.empty_like(ins[2]),
            torch.empty_like(ins[2]))
    ws = torch.empty(L.workspace_size("wkv4_backward", B, T, C), dtype=torch.uint8, device="cuda")
    g, _ = capture(lambda: L.wkv4_backward(*ins, out=outs, workspace=ws))
    for seed in (206, 207, 208):
        d = workloads.make_inputs(3, seed=seed, shape=(B, T, C))
        load(ins, [d[n] for n in ("w", "u", "k", "v", "gy")])
        g.replay()
        got = [host(t) for t in outs]
        eager = [host(t) for t in L.wkv4_backward(*ins)]
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), seed
        ref = oracle.wkv4_backward(d["w"], d["u"], d["k"], d["v"], d["gy"])
        errs = [rel_err(got[i], ref[i], None if i < 2 else 1) for i in range(4)]
        assert max(errs) <= TOL, (seed, errs)


def test_decay_adjoint_graph_replays(L):
    import torch
    B, T, C = 3, 3000, 96  # 24 slabs per row; glambda summed over slabs and rows
    announce("linrec_scan_real_decay_backward captured and replayed B=%d T=%d C=%d" % (B, T, C))

    def case(seed):
        d = workloads.make_gated(B, T, C, seed=seed, with_grad=True)
        x = oracle.scan_real_decay(d["lam"], d["h"], d["x0"]).astype(np.float32)
        return d, x

    d0, x0 = case(209)
    ins = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (d0["lam"], x0, d0["gx"], d0["x0"])]
    ws = torch.empty(L.workspace_size("scan_real_backward", B, T, C), dtype=torch.uint8, device="cuda")
    g, outs = capture(lambda: L.scan_real_decay_backward(*ins, want_gx0=True, workspace=ws))
    for seed in (210, 211, 212):
        d, x = case(seed)
        load(ins, (d["lam"], x, d["gx"], d["x0"]))
        g.replay()
        got = [host(t) for t in outs]
        eager = [host(t) for t in L.scan_real_decay_backward(*ins, want_gx0=True)]
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), seed
        ref = oracle.scan_real_decay_backward(d["lam"], x, d["gx"], d["x0"], want_gx0=True)
        errs = [rel_err(got[0], ref[0], None), rel_err(got[1], ref[1], 1), rel_err(got[2], ref[2], None)]
        assert max(errs) <= TOL, (seed, errs)


def test_ckpt_step_graph_replays(L):
    # The checkpointed training step captured whole: the forward's look-back and kept sums,
    # then the backward from them (RWKV-LLM page, eq. (14), "Time-mixing block", and its
    # chain rule).  10 forward slabs of 128 steps and 22 kept sums every 56.
    import torch
    B, T, C = 2, 1200, 130
    announce("wkv4_forward_ckpt + wkv4_backward_ckpt captured and replayed B=%d T=%d C=%d" % (B, T, C))
    d0 = workloads.make_inputs(3, seed=213, shape=(B, T, C))
    ins = [torch.from_numpy(d0[n]).cuda() for n in ("w", "u", "k", "v", "gy")]
    w, u, k, v, gy = ins
    lib = L.load()
    y = torch.empty_like(k)
    ck = torch.empty(L.wkv4_checkpoint_size(B, T, C), dtype=torch.uint8, device="cuda")
    fws = torch.empty(lib.wkv4_forward_ckpt_workspace_size(B, T, C), dtype=torch.uint8, device="cuda")
    bws = torch.empty(lib.wkv4_backward_ckpt_workspace_size(B, T, C), dtype=torch.uint8, device="cuda")
    outs = (torch.empty(C, device="cuda"), torch.empty(C, device="cuda"), torch.empty_like(k), torch.empty_like(k))

    def step():
        L.wkv4_forward_ckpt(w, u, k, v, out=(y, ck), workspace=fws)
        return L.wkv4_backward_ckpt(w, u, k, v, gy, ck, out=outs, workspace=bws)

    g, _ = capture(step)
    for seed in (214, 215, 216):
        d = workloads.make_inputs(3, seed=seed, shape=(B, T, C))
        load(ins, [d[n] for n in ("w", "u", "k", "v", "gy")])
        g.replay()
        got_y = host(y)
        got = [host(t) for t in outs]
        ey, eck = L.wkv4_forward_ckpt(w, u, k, v)
        eager = [host(t) for t in L.wkv4_backward_ckpt(w, u, k, v, gy, eck)]
        assert np.array_equal(got_y, host(ey)), seed
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), seed
        assert rel_err(got_y, oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL, seed
        ref = oracle.wkv4_backward(d["w"], d["u"], d["k"], d["v"], d["gy"])
        errs = [rel_err(got[i], ref[i], None if i < 2 else 1) for i in range(4)]
        assert max(errs) <= TOL, (seed, errs)
