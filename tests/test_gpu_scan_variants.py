"""GPU parity of the gated scan variants against the fp64 oracle, through the C ABI:
minGRU and minLSTM from gate pre-activations (minGRU page, minGRU and minLSTM sections), the
real scan with one decay per channel (LRU write-up, section on RWKV) and the LRU with
normalised input (LRU write-up, initialisation section).

Tolerance: 1e-4 relative, RMS-floored per sequence, as for the real scan (float32 carried
over long sequences; the gates add one sigmoid each, rounded to float32); 1e-3 for the
complex scan at T = 65536, as for the LRU workload.
"""

import math
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
    return t.cpu().numpy()


SHAPES = [(64, 4096, 256), (3, 333, 100), (2, 1, 64), (1, 5000, 40), (4, 777, 130)]


@pytest.mark.parametrize("with_x0", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_mingru(L, shape, with_x0):
    announce("linrec_scan_mingru %s x0=%s" % (shape, with_x0))
    d = workloads.make_gated(*shape, seed=70)
    x0 = d["x0"] if with_x0 else None
    got = host(L.scan_mingru(dev(d["kz"]), dev(d["h"]), dev(x0)))
    assert rel_err(got, oracle.scan_mingru(d["kz"], d["h"], x0)) <= TOL


@pytest.mark.parametrize("with_x0", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_minlstm(L, shape, with_x0):
    announce("linrec_scan_minlstm %s x0=%s" % (shape, with_x0))
    d = workloads.make_gated(*shape, seed=71)
    x0 = d["x0"] if with_x0 else None
    got = host(L.scan_minlstm(dev(d["kf"]), dev(d["ki"]), dev(d["h"]), dev(x0)))
    assert rel_err(got, oracle.scan_minlstm(d["kf"], d["ki"], d["h"], x0)) <= TOL


def test_gates_with_extreme_logits(L):
    """Logits of +-60: minGRU's 1 - z and minLSTM's normalised gates stay finite and exact
    where sigmoid saturates in float32."""
    announce("gated scans with logits ~ N(0, 30)")
    d = workloads.make_gated(3, 500, 96, seed=72, logit_std=30.0)
    got = host(L.scan_mingru(dev(d["kz"]), dev(d["h"]), dev(d["x0"])))
    assert np.all(np.isfinite(got))
    assert rel_err(got, oracle.scan_mingru(d["kz"], d["h"], d["x0"])) <= TOL
    got = host(L.scan_minlstm(dev(d["kf"]), dev(d["ki"]), dev(d["h"]), dev(d["x0"])))
    assert np.all(np.isfinite(got))
    assert rel_err(got, oracle.scan_minlstm(d["kf"], d["ki"], d["h"], d["x0"])) <= TOL


@pytest.mark.parametrize("with_x0", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_real_decay(L, shape, with_x0):
    announce("linrec_scan_real_decay %s x0=%s" % (shape, with_x0))
    d = workloads.make_gated(*shape, seed=73)
    x0 = d["x0"] if with_x0 else None
    lam = (0.5 + 0.5 * np.abs(d["lam"])).astype(np.float32)  # decays in [0.5, 1): long memory
    got = host(L.scan_real_decay(dev(lam), dev(d["h"]), dev(x0)))
    assert rel_err(got, oracle.scan_real_decay(lam, d["h"], x0)) <= TOL


@pytest.mark.parametrize("shape,tol", [((1, 65536, 256), 1e-3), ((4, 1000, 100), TOL), ((2, 1, 64), TOL),
                                       ((3, 3000, 33), TOL)], ids=str)
def test_complex_normalized(L, shape, tol):
    B, T, C = shape
    announce("linrec_scan_complex_normalized %s" % (shape,))
    lr = workloads.make_lru(B, T, C, 74)
    rng = np.random.default_rng(75)
    x0 = ((rng.standard_normal((B, C)) + 1j * rng.standard_normal((B, C))) / math.sqrt(2)).astype(np.complex64)
    got = host(L.scan_complex_normalized(dev(lr["lam"]), dev(lr["u"]), dev(x0)))
    assert rel_err(got, oracle.scan_complex_normalized(lr["lam"], lr["u"], x0)) <= tol


@pytest.mark.parametrize("shape", [(2, 700, 200), (1, 3000, 64), (3, 1, 40)], ids=str)
def test_complex_normalized_unit_circle(L, shape):
    """r = 1, the end of the LRU write-up's range r in [0, 1]: lambda = e^{i theta} stored
    as complex64.  Many such lambdas have |lambda|^2 a rounding above 1 (gamma = 0: the state
    rotates x0) and the rest a rounding below (gamma ~ 1e-4); both sides take gamma =
    sqrt(max(0, 1 - |lambda|^2)) from the same complex64 lambda."""
    B, T, C = shape
    announce("linrec_scan_complex_normalized unit circle %s" % (shape,))
    lr = workloads.make_lru(B, T, C, 86, 1.0, 1.0, 2 * math.pi, with_x0=True)
    lam = lr["lam"].copy()
    lam[:4] = np.array([1, -1, 1j, -1j], dtype=np.complex64)
    m2 = lam.real.astype(np.float64) ** 2 + lam.imag.astype(np.float64) ** 2  # exact squares, one rounding
    assert (m2 > 1.0).sum() >= C // 8 and (m2 < 1.0).sum() >= C // 8
    ref = oracle.scan_complex_normalized(lam, lr["u"], lr["x0"])
    assert np.all(np.isfinite(ref))
    got = host(L.scan_complex_normalized(dev(lam), dev(lr["u"]), dev(lr["x0"])))
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) <= TOL
    ref0 = oracle.scan_complex_normalized(lam, lr["u"])
    assert rel_err(host(L.scan_complex_normalized(dev(lam), dev(lr["u"]))), ref0) <= TOL


@pytest.mark.parametrize("vec", ["1", "2"])
def test_lane_widths(L, vec, monkeypatch):
    monkeypatch.setenv("LINREC_VEC", vec)
    announce("gated scans LINREC_VEC=%s" % vec)
    d = workloads.make_gated(4, 2000, 128, seed=76)
    assert rel_err(host(L.scan_mingru(dev(d["kz"]), dev(d["h"]), dev(d["x0"]))),
                   oracle.scan_mingru(d["kz"], d["h"], d["x0"])) <= TOL
    assert rel_err(host(L.scan_minlstm(dev(d["kf"]), dev(d["ki"]), dev(d["h"]), dev(d["x0"]))),
                   oracle.scan_minlstm(d["kf"], d["ki"], d["h"], d["x0"])) <= TOL
    assert rel_err(host(L.scan_real_decay(dev(d["lam"]), dev(d["h"]), dev(d["x0"]))),
                   oracle.scan_real_decay(d["lam"], d["h"], d["x0"])) <= TOL


def test_mingru_equals_materialised_scan(L):
    """The fused minGRU equals linrec_scan_real on a, b formed from the same gates (in
    float64, rounded once): the fusion changes where a, b are formed, not the scan."""
    announce("minGRU fused vs materialised")
    d = workloads.make_gated(8, 1500, 64, seed=77)
    z = 1.0 / (1.0 + np.exp(-d["kz"].astype(np.float64)))
    a, b = (1.0 - z).astype(np.float32), (z * d["h"]).astype(np.float32)
    fused = host(L.scan_mingru(dev(d["kz"]), dev(d["h"]), dev(d["x0"])))
    mat = host(L.scan_real(dev(a), dev(b), dev(d["x0"])))
    assert rel_err(fused, mat) <= 2 * TOL


def test_recompute_path(L, monkeypatch):
    """LINREC_SPIN=0: every look-back recomputes its predecessors from the inputs (the
    operators' per-step form, including the normalised input's scaling)."""
    monkeypatch.setenv("LINREC_SPIN", "0")
    announce("gated scans with LINREC_SPIN=0")
    d = workloads.make_gated(2, 3000, 64, seed=78)
    assert rel_err(host(L.scan_minlstm(dev(d["kf"]), dev(d["ki"]), dev(d["h"]), dev(d["x0"]))),
                   oracle.scan_minlstm(d["kf"], d["ki"], d["h"], d["x0"])) <= TOL
    lr = workloads.make_lru(1, 20000, 64, 79)
    assert rel_err(host(L.scan_complex_normalized(dev(lr["lam"]), dev(lr["u"]))),
                   oracle.scan_complex_normalized(lr["lam"], lr["u"])) <= 1e-3
