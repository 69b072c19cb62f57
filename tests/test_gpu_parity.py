"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Tolerance (RMS-floored maximum relative error, see ``oracle.compare``): 1e-4 for float32
results, 1e-3 for the complex64 LRU scan at T = 262144 (the bounds the workloads are
specified with).  Every call goes through the C ABI via the ctypes binding.
"""

import os
import sys

import numpy as np
import pytest

import oracle
from oracle.compare import chan_ratio, plain_rel, rel_err
from linear_recurrence_rnn_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_LRU = 1e-3


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


def gpu_wkv(L, d):
    y = L.wkv4_forward(dev(d["w"]), dev(d["u"]), dev(d["k"]), dev(d["v"]))
    return host(y)


def gpu_wkv_bwd(L, d):
    outs = L.wkv4_backward(dev(d["w"]), dev(d["u"]), dev(d["k"]), dev(d["v"]), dev(d["gy"]))
    return [host(t) for t in outs]


def worst(out, ref, time_axis=1):
    """Index, value and reference of the element with the largest floored relative error."""
    mag = np.abs(ref)
    floor = np.sqrt(np.mean(mag * mag)) if time_axis is None else \
        np.sqrt(np.mean(mag * mag, axis=time_axis, keepdims=True))
    e = np.abs(out - ref) / np.maximum(np.maximum(mag, floor), 1e-30)
    i = np.unravel_index(int(np.argmax(e)), e.shape)
    return {"index": tuple(int(x) for x in i), "got": float(out[i]), "ref": float(ref[i])}


def ref_bwd(d):
    """The oracle's (gw, gu, gk, gv) and the conditioning sums (cw, cu) of gw and gu."""
    r = oracle.wkv4_backward_cond(d["w"], d["u"], d["k"], d["v"], d["gy"])
    return list(r[:4]), (r[6], r[7])


def check_bwd(got, ref, cond=None, tol=TOL):
    """Parity of (gw, gu, gk, gv).  gk, gv: RMS-floored per sequence.  gw, gu: RMS-floored
    over channels and, given their conditioning sums cond = (cw, cu), channel by channel:
    |err_c| <= max(tol |ref_c|, 2^-20 cond_c) (the plain per-channel relative error is
    reported alongside)."""
    gw, gu, gk, gv = got
    rw, ru, rk, rv = ref
    T = gk.shape[1]
    errs = {"gk": rel_err(gk, rk), "gv": rel_err(gv, rv)}
    if T == 1:
        # One step: y_0 = v_0 exactly, so dL/dw = dL/du = 0 and dL/dk_0 = 0 (no later step
        # feeds G or H); the oracle's values are its own rounding noise (~1e-16), so
        # compare absolutely, dL/dk against a bound far below any real value.
        errs["gw"] = float(np.max(np.abs(gw - rw)))
        errs["gu"] = float(np.max(np.abs(gu - ru)))
        errs["gk"] = float(np.max(np.abs(gk - rk))) * (TOL / 1e-6)
    else:
        errs["gw"] = rel_err(gw, rw, None)
        errs["gu"] = rel_err(gu, ru, None)
    detail = {k: worst(o, r, None if k in ("gw", "gu") else 1)
              for k, o, r in (("gw", gw, rw), ("gu", gu, ru), ("gk", gk, rk), ("gv", gv, rv))
              if errs[k] > tol}
    assert all(e <= tol for e in errs.values()), (errs, detail)
    if cond is not None:
        chan = {"gw": chan_ratio(gw, rw, cond[0], tol), "gu": chan_ratio(gu, ru, cond[1], tol)}
        plain = {"gw": plain_rel(gw, rw), "gu": plain_rel(gu, ru)}
        assert all(v <= 1.0 for v in chan.values()), (chan, plain)
    return errs


# ---------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("wid", [1, 2])
def test_wkv_forward_workloads(L, wid):
    announce("wkv4_forward workload %d %s" % (wid, workloads.WORKLOADS[wid].label))
    d = workloads.make_inputs(wid)
    err = rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"]))
    assert err <= TOL, err


@pytest.fixture(scope="module")
def wl3():
    return workloads.make_inputs(3)


def test_wkv_workload3_forward(L, wl3):
    announce("wkv4_forward workload 3 B=8 T=4096 C=2560")
    d = wl3
    err = rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"]))
    assert err <= TOL, err


def test_wkv_workload3_backward(L, wl3):
    announce("wkv4_backward workload 3 B=8 T=4096 C=2560")
    d = wl3
    got = gpu_wkv_bwd(L, d)
    ref, cond = ref_bwd(d)
    check_bwd(got, ref, cond)


def test_scan_real_workload4(L):
    announce("linrec_scan_real workload 4 B=64 T=4096 C=256")
    d = workloads.make_inputs(4)
    x = host(L.scan_real(dev(d["a"]), dev(d["b"])))
    err = rel_err(x, oracle.scan_real(d["a"], d["b"]))
    assert err <= TOL, err


def test_scan_complex_workload5(L):
    announce("linrec_scan_complex workload 5 B=1 T=262144 C=1024")
    d = workloads.make_inputs(5)
    x = host(L.scan_complex(dev(d["lam"]), dev(d["u"])))
    ref = oracle.scan_complex(d["lam"], d["u"])
    err = rel_err(x, ref)
    del ref
    assert err <= TOL_LRU, err


# ---------------------------------------------------------------- shapes and edge cases
WKV_SHAPES = [(1, 1, 4), (3, 1000, 40), (2, 333, 37), (1, 17, 1), (4, 2049, 20), (2, 64, 16)]


@pytest.mark.parametrize("shape", WKV_SHAPES, ids=[str(s) for s in WKV_SHAPES])
def test_wkv_forward_shapes(L, shape):
    announce("wkv4_forward shape %s" % (shape,))
    d = workloads.make_inputs(3, seed=7, shape=shape)
    err = rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"]))
    assert err <= TOL, err


@pytest.mark.parametrize("shape", WKV_SHAPES, ids=[str(s) for s in WKV_SHAPES])
def test_wkv_backward_shapes(L, shape):
    announce("wkv4_backward shape %s" % (shape,))
    d = workloads.make_inputs(3, seed=8, shape=shape)
    check_bwd(gpu_wkv_bwd(L, d), *ref_bwd(d))


def test_wkv_unaligned_views(L):
    # Views offset by one float: the library must take its scalar (4-byte) path.
    import torch
    announce("wkv4_forward/backward unaligned views B=2 T=300 C=24")
    B, T, C = 2, 300, 24
    d = workloads.make_inputs(3, seed=9, shape=(B, T, C))

    def shifted(x):
        buf = torch.empty(x.size + 1, dtype=torch.float32, device="cuda")
        t = buf[1:].view(x.shape)
        t.copy_(torch.from_numpy(x))
        return t

    k, v, gy = shifted(d["k"]), shifted(d["v"]), shifted(d["gy"])
    y = host(L.wkv4_forward(dev(d["w"]), dev(d["u"]), k, v, out=shifted(np.zeros_like(d["k"]))))
    assert rel_err(y, oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL
    outs = L.wkv4_backward(dev(d["w"]), dev(d["u"]), k, v, gy,
                           out=(dev(np.zeros(C, np.float32)), dev(np.zeros(C, np.float32)),
                                shifted(np.zeros_like(d["k"])), shifted(np.zeros_like(d["k"]))))
    check_bwd([host(t) for t in outs], *ref_bwd(d))


def test_wkv_stress_spikes(L):
    announce("wkv4_forward/backward k spikes +-150, w in {0, 1e4}")
    B, T, C = 2, 700, 32
    d = workloads.make_inputs(3, seed=10, shape=(B, T, C))
    d["k"][0, 100, :] = 150.0
    d["k"][1, 350, 3] = -150.0
    d["k"][1, 20:40, 5] = 120.0
    d["w"][0] = 0.0
    d["w"][1] = 1e4
    err = rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"]))
    assert err <= TOL, err
    check_bwd(gpu_wkv_bwd(L, d), *ref_bwd(d))


@pytest.mark.parametrize("wid", [2, 3])
def test_wkv_exact_path_matches_fast_path(L, monkeypatch, wid):
    # The per-chunk frame (one exponential per element) and the exact per-step running
    # maximum must agree; both against the oracle.
    announce("wkv4_forward exact-only path vs default, workload %d shape" % wid)
    d = workloads.make_inputs(wid, seed=21, shape=(2, 1500, 96))
    ref = oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])
    y_fast = gpu_wkv(L, d)
    monkeypatch.setenv("LINREC_WKV_EXACT", "1")
    y_exact = gpu_wkv(L, d)
    assert rel_err(y_fast, ref) <= TOL and rel_err(y_exact, ref) <= TOL
    assert rel_err(y_fast, y_exact.astype(np.float64)) <= 2 * TOL


SHAPES_NW_L_VEC = [(nw, lc, vec) for (nw, lc) in [("4", "16"), ("8", "8"), ("8", "16")]
                   for vec in ("4", "2", "1")] + [("8", "32", "1")]


@pytest.mark.parametrize("nw,lc,vec", SHAPES_NW_L_VEC, ids=["nw%s_L%s_vec%s" % x for x in SHAPES_NW_L_VEC])
def test_forward_launch_shapes(L, monkeypatch, nw, lc, vec):
    # Every kernel shape (waves per slab x steps per chunk) against the oracle, with ragged
    # slabs, partial channel groups and the scalar (vec 1) variant.  (8, 32) exists for the
    # linear scans only; WKV then runs its default shape.
    announce("forward launch shape nw=%s L=%s vec<=%s" % (nw, lc, vec))
    monkeypatch.setenv("LINREC_NW", nw)
    monkeypatch.setenv("LINREC_L", lc)
    monkeypatch.setenv("LINREC_VEC", vec)
    d = workloads.make_inputs(3, seed=11, shape=(2, 1000, 296))
    assert rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL
    r = workloads.make_inputs(4, seed=11, shape=(3, 777, 260))
    x0 = np.random.default_rng(3).standard_normal((3, 260)).astype(np.float32)
    assert rel_err(host(L.scan_real(dev(r["a"]), dev(r["b"]), dev(x0))), oracle.scan_real(r["a"], r["b"], x0)) <= TOL
    c = workloads.make_inputs(5, seed=11, shape=(2, 900, 130))
    assert rel_err(host(L.scan_complex(dev(c["lam"]), dev(c["u"]))), oracle.scan_complex(c["lam"], c["u"])) <= TOL
    # Short sequences: chains of at most 1 + KB slabs (KB = 8, 4 or 2 records in flight for
    # 1, 2 or 4 channels per lane) publish aggregates only.
    d = workloads.make_inputs(3, seed=12, shape=(2, 300, 296))
    assert rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL
    r = workloads.make_inputs(4, seed=12, shape=(3, 250, 260))
    x0 = np.random.default_rng(5).standard_normal((3, 260)).astype(np.float32)
    assert rel_err(host(L.scan_real(dev(r["a"]), dev(r["b"]), dev(x0))), oracle.scan_real(r["a"], r["b"], x0)) <= TOL


@pytest.mark.parametrize("spin", ["0", "1"])
def test_lookback_recompute_path(L, monkeypatch, spin):
    # With no (or one) poll of a predecessor's flag, the waiting wave recomputes the
    # predecessor slab's aggregate from its inputs: results must not change.
    announce("forward look-back with LINREC_SPIN=%s" % spin)
    monkeypatch.setenv("LINREC_SPIN", spin)
    d = workloads.make_inputs(3, seed=12, shape=(2, 1500, 512))
    assert rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL
    r = workloads.make_inputs(4, seed=12, shape=(2, 1500, 256))
    x0 = np.random.default_rng(4).standard_normal((2, 256)).astype(np.float32)
    assert rel_err(host(L.scan_real(dev(r["a"]), dev(r["b"]), dev(x0))), oracle.scan_real(r["a"], r["b"], x0)) <= TOL
    c = workloads.make_inputs(5, seed=12, shape=(1, 3000, 128))
    xc0 = (np.ones((1, 128)) + 0.5j).astype(np.complex64)
    assert rel_err(host(L.scan_complex(dev(c["lam"]), dev(c["u"]), dev(xc0))),
                   oracle.scan_complex(c["lam"], c["u"], xc0)) <= TOL
    # Short chains (at most 9 slabs of 128 steps: aggregates only) take the same fallback.
    d = workloads.make_inputs(3, seed=13, shape=(2, 1100, 320))
    assert rel_err(gpu_wkv(L, d), oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL
    r = workloads.make_inputs(4, seed=13, shape=(2, 1000, 256))
    assert rel_err(host(L.scan_real(dev(r["a"]), dev(r["b"]), dev(x0))), oracle.scan_real(r["a"], r["b"], x0)) <= TOL


@pytest.mark.parametrize("wid", [2, 3])
def test_backward_exact_path_matches_fast_path(L, monkeypatch, wid):
    # The backward's per-chunk frame (no exponential in the reverse) and its exact per-step
    # path must agree; both against the oracle.
    announce("wkv4_backward exact-only path vs default, workload %d shape" % wid)
    d = workloads.make_inputs(wid, seed=22, shape=(2, 1500, 96))
    if "gy" not in d:
        d["gy"] = np.random.default_rng(5).standard_normal(d["k"].shape).astype(np.float32)
    ref, cond = ref_bwd(d)
    fast = gpu_wkv_bwd(L, d)
    monkeypatch.setenv("LINREC_WKV_EXACT", "1")
    exact = gpu_wkv_bwd(L, d)
    check_bwd(fast, ref, cond)
    check_bwd(exact, ref, cond)
    for name, a, b in zip(("gw", "gu", "gk", "gv"), fast, exact):
        ax = None if name in ("gw", "gu") else 1
        assert rel_err(a, b.astype(np.float64), ax) <= 2 * TOL, name


BWD_SHAPES_NW_L = [("3", "16"), ("4", "16"), ("7", "8"), ("8", "8"), ("7", "16")]


@pytest.mark.parametrize("nw,lc", BWD_SHAPES_NW_L, ids=["nw%s_L%s" % x for x in BWD_SHAPES_NW_L])
def test_backward_launch_shapes(L, monkeypatch, nw, lc):
    # Every backward kernel shape against the oracle: ragged last slab, a partial channel
    # group, and a sequence that fits one slab.
    announce("backward launch shape nw=%s L=%s" % (nw, lc))
    monkeypatch.setenv("LINREC_BWD_NW", nw)
    monkeypatch.setenv("LINREC_BWD_L", lc)
    for shape in [(2, 1001, 150), (3, 40, 70)]:
        d = workloads.make_inputs(3, seed=13, shape=shape)
        check_bwd(gpu_wkv_bwd(L, d), *ref_bwd(d))


@pytest.mark.parametrize("spin", ["0", "1"])
def test_backward_lookback_recompute_path(L, monkeypatch, spin):
    # With no (or one) poll, both the forward-state chain and the reverse chain recompute
    # the records of slabs that have not published from their inputs.
    announce("backward look-back with LINREC_SPIN=%s" % spin)
    monkeypatch.setenv("LINREC_SPIN", spin)
    d = workloads.make_inputs(3, seed=14, shape=(2, 1300, 130))
    d["k"][1, 600, 7] = 140.0
    check_bwd(gpu_wkv_bwd(L, d), *ref_bwd(d))


def test_backward_long_single_sequence(L):
    # Many slabs in one chain (look-back windows of more than 64 slabs).
    announce("wkv4_backward B=1 T=20000 C=64")
    d = workloads.make_inputs(3, seed=15, shape=(1, 20000, 64))
    check_bwd(gpu_wkv_bwd(L, d), *ref_bwd(d))


def test_forward_determinism_and_vec1(L, monkeypatch):
    announce("wkv4_forward run twice; default width vs 4 channels per lane B=3 T=2000 C=256")
    d = workloads.make_inputs(2, seed=12, shape=(3, 2000, 256))
    ref = oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])
    y1 = gpu_wkv(L, d)
    y2 = gpu_wkv(L, d)
    np.testing.assert_array_equal(y1, y2)
    monkeypatch.setenv("LINREC_VEC", "4")
    y3 = gpu_wkv(L, d)
    assert rel_err(y1, ref) <= TOL and rel_err(y3, ref) <= TOL
    g1 = gpu_wkv_bwd(L, workloads.make_inputs(3, seed=12, shape=(3, 700, 64)))
    g2 = gpu_wkv_bwd(L, workloads.make_inputs(3, seed=12, shape=(3, 700, 64)))
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(a, b)


def test_wkv_backward_empty_batch(L):
    import torch
    announce("wkv4_backward B=0 zero gw, gu")
    C = 12
    w = dev(np.ones(C, np.float32))
    z = torch.empty((0, 5, C), dtype=torch.float32, device="cuda")
    gw, gu, gk, gv = L.wkv4_backward(w, w, z, z, z)
    np.testing.assert_array_equal(host(gw), 0.0)
    np.testing.assert_array_equal(host(gu), 0.0)


REAL_SHAPES = [(1, 1, 4), (3, 1000, 40), (2, 333, 37), (5, 50, 3)]


@pytest.mark.parametrize("shape", REAL_SHAPES, ids=[str(s) for s in REAL_SHAPES])
@pytest.mark.parametrize("with_x0", [False, True])
def test_scan_real_shapes(L, shape, with_x0):
    announce("linrec_scan_real shape %s x0=%s" % (shape, with_x0))
    d = workloads.make_inputs(4, seed=13, shape=shape)
    x0 = np.random.default_rng(1).standard_normal((shape[0], shape[2])).astype(np.float32) if with_x0 else None
    x = host(L.scan_real(dev(d["a"]), dev(d["b"]), None if x0 is None else dev(x0)))
    assert rel_err(x, oracle.scan_real(d["a"], d["b"], x0)) <= TOL


CPLX_SHAPES = [(1, 1, 2), (2, 777, 33), (3, 4096, 64), (1, 20000, 8)]


@pytest.mark.parametrize("shape", CPLX_SHAPES, ids=[str(s) for s in CPLX_SHAPES])
def test_scan_complex_shapes(L, shape):
    announce("linrec_scan_complex shape %s" % (shape,))
    d = workloads.make_inputs(5, seed=16, shape=shape)
    x = host(L.scan_complex(dev(d["lam"]), dev(d["u"])))
    assert rel_err(x, oracle.scan_complex(d["lam"], d["u"])) <= TOL


def test_complex_zero_phase_matches_real_scan(L):
    announce("linrec_scan_complex theta=0 vs linrec_scan_real")
    d = workloads.make_lru(2, 1500, 24, 17, theta_hi=0.0)
    xc = host(L.scan_complex(dev(d["lam"]), dev(d["u"])))
    a = np.ascontiguousarray(np.broadcast_to(d["lam"].real[None, None, :], d["u"].shape)).astype(np.float32)
    xr = host(L.scan_real(dev(a), dev(np.ascontiguousarray(d["u"].real))))
    xi = host(L.scan_real(dev(a), dev(np.ascontiguousarray(d["u"].imag))))
    assert rel_err(xc.real, xr) <= 1e-5 and rel_err(xc.imag, xi) <= 1e-5


def test_scan_special_cases(L):
    announce("linrec_scan_real a=1 cumsum, a=0 copy")
    rng = np.random.default_rng(18)
    b = rng.standard_normal((2, 900, 12)).astype(np.float32)
    x = host(L.scan_real(dev(np.ones_like(b)), dev(b)))
    assert rel_err(x, np.cumsum(b.astype(np.float64), axis=1)) <= TOL
    x = host(L.scan_real(dev(np.zeros_like(b)), dev(b)))
    np.testing.assert_array_equal(x, b)


def test_flat_grid_matches_3d_grid(L, monkeypatch):
    # The scan kernels and the WKV gradient kernel run on a 3-D grid (channel groups, batch
    # rows, slabs) whenever the rows and slabs fit its y and z extents, and on a flat grid,
    # whose block index is divided into the same three, otherwise.  Both number the blocks
    # alike, so the results must agree bit for bit (forward WKV, real and complex scans, a
    # reverse-time adjoint, the WKV backward), and with the oracle.
    announce("flat grid (LINREC_FLAT_GRID=1) vs 3-D grid")
    d = workloads.make_inputs(3, seed=31, shape=(3, 1100, 200))
    r = workloads.make_inputs(4, seed=31, shape=(3, 900, 260))
    c = workloads.make_inputs(5, seed=31, shape=(2, 1300, 130))
    gx = np.random.default_rng(31).standard_normal(r["a"].shape).astype(np.float32)

    def run():
        y = gpu_wkv(L, d)
        xr = L.scan_real(dev(r["a"]), dev(r["b"]))
        ga, gb, _ = L.scan_real_backward(dev(r["a"]), xr, dev(gx))
        xc = host(L.scan_complex(dev(c["lam"]), dev(c["u"])))
        return [y, host(xr), host(ga), host(gb), xc] + gpu_wkv_bwd(L, d)

    base = run()
    monkeypatch.setenv("LINREC_FLAT_GRID", "1")
    flat = run()
    for a, f in zip(base, flat):
        assert a.tobytes() == f.tobytes()
    assert rel_err(flat[0], oracle.wkv4_forward(d["w"], d["u"], d["k"], d["v"])) <= TOL
    assert rel_err(flat[1], oracle.scan_real(r["a"], r["b"])) <= TOL
    assert rel_err(flat[4], oracle.scan_complex(c["lam"], c["u"])) <= TOL
