"""Host-only checks of the C ABI: the library loads, exports every function that
``include/linrec.h`` declares, and rejects bad arguments before making any HIP call.

No kernel is launched here: every call below returns from the host-side checks.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linrec.h")
LIB = os.path.join(ROOT, "linear_recurrence_rnn_amd", "liblinrec.so")

OK, INVALID, WORKSPACE, UNSUPPORTED, HIPERR = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("liblinrec.so is not built (run python -m linear_recurrence_rnn_amd.build)")
    from linear_recurrence_rnn_amd import binding
    return binding.load()


def test_header_declares_the_four_operations():
    names = declared_functions()
    for n in ("wkv4_forward", "wkv4_backward", "linrec_scan_real", "linrec_scan_complex",
              "wkv4_forward_workspace_size", "wkv4_backward_workspace_size",
              "linrec_scan_workspace_size", "linrec_abi_version", "linrec_status_string",
              "linrec_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_the_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(declared_functions())


def test_version_and_status_strings(lib):
    m = re.search(r"#define LINREC_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.linrec_abi_version() == int(m.group(1))
    assert lib.linrec_status_string(OK) == b"LINREC_OK"
    assert lib.linrec_status_string(WORKSPACE) == b"LINREC_ERR_WORKSPACE"
    assert lib.linrec_status_string(99) == b"unknown status"


P = ctypes.c_void_p(0x100000)       # aligned fake device addresses: never dereferenced
P2 = ctypes.c_void_p(0x200000)
ODD = ctypes.c_void_p(0x100002)     # not 4-byte aligned


def fwd(lib, B, T, C, ptrs=None, ws=None, nws=0):
    w, u, k, v, y = ptrs or (P, P, P, P, P2)
    return lib.wkv4_forward(B, T, C, w, u, k, v, y, ws, nws, None)


def test_negative_and_overflowing_sizes(lib):
    assert fwd(lib, -1, 4, 4) == INVALID
    assert b"negative" in lib.linrec_last_error()
    assert fwd(lib, 4, -2, 4) == INVALID
    assert fwd(lib, 1 << 31, 1 << 31, 1 << 10) == INVALID
    assert b"overflow" in lib.linrec_last_error()
    assert lib.linrec_scan_real(-1, 1, 1, P, P, None, P2, None, 0, None) == INVALID
    assert lib.linrec_scan_complex(1, 1 << 40, 1 << 30, P, P, None, P2, None, 0, None) == INVALID
    assert lib.wkv4_backward(1, -1, 1, P, P, P, P, P, P2, P2, P2, P2, None, 0, None) == INVALID


def test_null_pointers(lib):
    assert fwd(lib, 1, 4, 4, (P, None, P, P, P2)) == INVALID
    assert b"NULL" in lib.linrec_last_error()
    assert lib.linrec_scan_real(1, 4, 4, P, None, None, P2, None, 0, None) == INVALID
    assert lib.linrec_scan_complex(1, 4, 4, None, P, None, P2, None, 0, None) == INVALID
    assert lib.wkv4_backward(1, 4, 4, P, P, P, P, None, P2, P2, P2, P2, None, 0, None) == INVALID


def test_empty_shapes_are_noops(lib):
    # Forward and scans enqueue nothing for an empty shape.
    assert fwd(lib, 0, 16, 16) == OK
    assert fwd(lib, 2, 0, 16) == OK
    assert fwd(lib, 2, 16, 0) == OK
    assert lib.linrec_scan_real(0, 4, 4, P, P, None, P2, None, 0, None) == OK
    assert lib.linrec_scan_complex(3, 0, 4, P, P, None, P2, None, 0, None) == OK
    assert lib.wkv4_backward(2, 5, 0, P, P, P, P, P, P2, P2, P2, P2, None, 0, None) == OK


def test_misaligned_pointers(lib):
    assert fwd(lib, 1, 4, 4, (P, P, ODD, P, P2)) == UNSUPPORTED
    assert b"aligned" in lib.linrec_last_error()
    # complex64 needs 8-byte alignment
    assert lib.linrec_scan_complex(1, 4, 4, P, ctypes.c_void_p(0x100004), None, P2, None, 0,
                                   None) == UNSUPPORTED


def test_workspace_checks(lib):
    # A single long sequence is cut into slabs and needs workspace.
    B, T, C = 1, 262144, 1024
    need = lib.linrec_scan_workspace_size(B, T, C, 1)
    assert need > 0
    assert lib.linrec_scan_complex(B, T, C, P, P, None, P2, None, 0, None) == WORKSPACE
    assert lib.linrec_scan_complex(B, T, C, P, P, None, P2, None, need, None) == INVALID  # NULL ws
    assert lib.linrec_scan_complex(B, T, C, P, P, None, P2, ctypes.c_void_p(0x300008), need,
                                   None) == UNSUPPORTED  # not 16-byte aligned
    assert lib.wkv4_backward_workspace_size(8, 4096, 2560) > 0
    need_b = lib.wkv4_backward_workspace_size(2, 100, 8)
    assert lib.wkv4_backward(2, 100, 8, P, P, P, P, P, P2, P2, P2, P2, None, need_b - 1,
                             None) == WORKSPACE


def test_workspace_sizes(lib):
    assert lib.wkv4_forward_workspace_size(0, 10, 10) == 0
    assert lib.wkv4_forward_workspace_size(-1, 10, 10) == 0
    # A sequence that fits one time slab needs no look-back records.
    assert lib.wkv4_forward_workspace_size(1, 64, 32) == 0
    assert lib.linrec_scan_workspace_size(3, 40, 500, 1) == 0
    # Longer sequences need per-slab flags and records; more slabs need more.
    w1 = lib.wkv4_forward_workspace_size(8, 1024, 768)
    w2 = lib.wkv4_forward_workspace_size(8, 2048, 768)
    assert 0 < w1 < w2
    assert lib.linrec_scan_workspace_size(64, 4096, 256, 0) > 0
    assert lib.linrec_scan_workspace_size(1, 1 << 16, 64, 1) > 0


def test_scan_backward_argument_checks(lib):
    rb, cb = lib.linrec_scan_real_backward, lib.linrec_scan_complex_backward
    # null required pointers
    assert rb(1, 4, 4, P, None, None, P, P2, P2, None, None, 0, None) == INVALID
    assert cb(1, 4, 4, P, None, P, P, None, P2, None, None, 0, None) == INVALID  # glambda NULL
    assert cb(1, 4, 4, None, None, P, P, P2, P2, None, None, 0, None) == INVALID
    # empty shapes without outputs to fill: nothing enqueued
    assert rb(0, 4, 4, P, None, P, P, P2, P2, P2, None, 0, None) == OK
    assert rb(2, 0, 4, P, None, P, P, P2, P2, None, None, 0, None) == OK
    assert cb(2, 3, 0, P, None, P, P, P2, P2, None, None, 0, None) == OK
    # alignment: complex64 needs 8 bytes
    assert cb(1, 4, 4, P, None, ctypes.c_void_p(0x100004), P, P2, P2, None, None, 0, None) == UNSUPPORTED
    assert rb(1, 4, 4, ODD, None, P, P, P2, P2, None, None, 0, None) == UNSUPPORTED
    # workspace: a long single sequence needs look-back records
    need = lib.linrec_scan_backward_workspace_size(1, 1 << 16, 64, 1)
    assert need > 0
    assert cb(1, 1 << 16, 64, P, None, P, P, P2, P2, None, P, 16, None) == WORKSPACE
    # the complex adjoints always need room for their per-slab sums of glambda; so does the
    # real family's query, which covers the per-channel decay's adjoint
    assert lib.linrec_scan_backward_workspace_size(2, 40, 8, 1) > 0
    assert lib.linrec_scan_backward_workspace_size(2, 40, 8, 0) > 0


def test_variant_backward_argument_checks(lib):
    mg, ml = lib.linrec_scan_mingru_backward, lib.linrec_scan_minlstm_backward
    rd, cn = lib.linrec_scan_real_decay_backward, lib.linrec_scan_complex_normalized_backward
    # (B, T, C, ins..., x0, x, gx, outs..., gx0, ws, bytes, stream)
    assert mg(2, 8, 4, P, None, None, P, P, P2, P2, None, P, 1 << 20, None) == INVALID       # h NULL
    assert ml(2, 8, 4, P, P, P, None, P, P, P2, None, P2, None, P, 1 << 20, None) == INVALID  # gki NULL
    assert mg(2, 8, 4, P, P, None, P, ODD, P2, P2, None, P, 1 << 20, None) == UNSUPPORTED
    assert mg(2, 8, 4, P, P, ODD, P, P, P2, P2, None, P, 1 << 20, None) == UNSUPPORTED     # x0
    # empty shapes: nothing to do without outputs to fill
    assert mg(0, 8, 4, P, P, None, P, P, P2, P2, None, None, 0, None) == OK
    assert ml(2, 8, 0, P, P, P, None, P, P, P2, P2, P2, None, None, 0, None) == OK
    # the decay's adjoint needs glambda; complex64 pointers need 8 bytes
    assert rd(2, 8, 4, P, None, P, P, None, P2, None, P, 1 << 20, None) == INVALID
    assert rd(2, 8, 4, P, None, P, P, ODD, P2, None, P, 1 << 20, None) == UNSUPPORTED
    assert cn(2, 8, 4, P, None, None, P, P, P2, P2, None, P, 1 << 20, None) == INVALID      # u NULL
    assert cn(2, 8, 4, P, P, None, P, P, ctypes.c_void_p(0x200004), P2, None, P, 1 << 20, None) == UNSUPPORTED
    # workspace
    need = lib.linrec_scan_backward_workspace_size(1, 1 << 14, 64, 0)
    assert need > 0
    assert rd(1, 1 << 14, 64, P, None, P, P, P2, P2, None, P, 16, None) == WORKSPACE
    assert cn(1, 1 << 14, 64, P, P, None, P, P, P2, P2, None, P, 16, None) == WORKSPACE


def test_wkv4_forward_ex_argument_checks(lib):
    fx = lib.wkv4_forward_ex
    # empty batch / channels: nothing to do
    assert fx(0, 4, 4, P, P, P, P, None, None, P2, None, None, 0, None) == OK
    # no tokens and no state out: nothing to do
    assert fx(2, 0, 4, P, P, P, P, None, None, P2, None, None, 0, None) == OK
    # required pointers
    assert fx(1, 4, 4, None, P, P, P, None, None, P2, None, None, 0, None) == INVALID
    assert fx(1, 4, 4, P, P, P, P, None, None, None, None, None, 0, None) == INVALID
    # misaligned optional inputs
    assert fx(1, 4, 4, P, P, P, P, ODD, None, P2, None, None, 0, None) == UNSUPPORTED
    assert fx(1, 4, 4, P, P, P, P, None, ODD, P2, None, None, 0, None) == UNSUPPORTED


def test_wkv4_decode_step_argument_checks(lib):
    fd = lib.wkv4_decode_step
    # empty batch / channels: nothing to do, no pointer read
    assert fd(0, 4, None, None, None, None, None, None, None, None) == OK
    assert fd(3, 0, None, None, None, None, None, None, None, None) == OK
    assert fd(-1, 4, P, P, P, P, None, P2, P2, None) == INVALID
    # B * 3 * C floats overflowing int64
    assert fd(1 << 40, 1 << 40, P, P, P, P, None, P2, P2, None) == INVALID
    # required pointers (r is optional)
    for i in (0, 1, 2, 3, 5, 6):
        args = [P, P, P, P, None, P2, P2]
        args[i] = None
        assert fd(2, 4, *args, None) == INVALID, i
    # alignment of every pointer, the optional gate included
    for i in range(7):
        args = [P, P, P, P, P, P2, P2]
        args[i] = ODD
        assert fd(2, 4, *args, None) == UNSUPPORTED, i


def test_token_shift_argument_checks(lib):
    f, fb, wsz = lib.rwkv_token_shift, lib.rwkv_token_shift_backward, lib.rwkv_token_shift_backward_workspace_size
    # empty shapes: nothing to do, no pointer read
    assert f(0, 4, 4, 3, None, None, None, None, None) == OK
    assert f(2, 0, 4, 3, None, None, None, None, None) == OK
    # M outside 1..4, negative sizes, overflow
    assert f(1, 4, 4, 0, P, None, P, P2, None) == INVALID
    assert f(1, 4, 4, 5, P, None, P, P2, None) == INVALID
    assert f(-1, 4, 4, 3, P, None, P, P2, None) == INVALID
    assert f(1 << 40, 1 << 20, 4, 3, P, None, P, P2, None) == INVALID
    # required pointers, alignment (x_prev optional)
    assert f(1, 4, 4, 3, None, None, P, P2, None) == INVALID
    assert f(1, 4, 4, 3, P, None, P, None, None) == INVALID
    assert f(1, 4, 4, 3, P, ODD, P, P2, None) == UNSUPPORTED
    assert f(1, 4, 4, 3, P, None, ODD, P2, None) == UNSUPPORTED
    # backward: workspace size and checks
    need = wsz(2, 100, 8, 3)
    assert need > 0 and wsz(2, 0, 8, 3) == 0 and wsz(2, 100, 8, 7) == 0
    assert fb(2, 100, 8, 3, P, None, P, P, P2, P2, None, None, need, None) == INVALID   # NULL workspace
    assert fb(2, 100, 8, 3, P, None, P, P, P2, P2, None, P, need - 1, None) == WORKSPACE
    assert fb(2, 100, 8, 3, P, None, P, None, P2, P2, None, P, need, None) == INVALID
    assert fb(2, 100, 8, 3, P, None, P, P, P2, ODD, None, P, need, None) == UNSUPPORTED
    assert fb(2, 100, 8, 9, P, None, P, P, P2, P2, None, P, need, None) == INVALID
    assert fb(2, 100, 0, 3, None, None, None, None, None, None, None, None, 0, None) == OK
    # empty batch or sequence needs gmu to zero-fill
    assert fb(2, 0, 8, 3, None, None, None, None, None, None, None, None, 0, None) == INVALID


def test_gated_scan_argument_checks(lib):
    need = lib.linrec_scan_workspace_size(2, 1 << 12, 64, 0)
    needc = lib.linrec_scan_workspace_size(2, 1 << 12, 64, 1)
    for name, nin in (("linrec_scan_mingru", 2), ("linrec_scan_minlstm", 3), ("linrec_scan_real_decay", 2)):
        f = getattr(lib, name)
        ins = [P] * nin
        assert f(0, 4, 4, *[None] * nin, None, None, None, 0, None) == OK, name
        assert f(-1, 4, 4, *ins, None, P2, None, 0, None) == INVALID, name
        for i in range(nin):
            bad = list(ins)
            bad[i] = None
            assert f(2, 1 << 12, 64, *bad, None, P2, P, need, None) == INVALID, (name, i)
            bad[i] = ODD
            assert f(2, 1 << 12, 64, *bad, None, P2, P, need, None) == UNSUPPORTED, (name, i)
        assert f(2, 1 << 12, 64, *ins, None, None, P, need, None) == INVALID, name
        assert f(2, 1 << 12, 64, *ins, ODD, P2, P, need, None) == UNSUPPORTED, name
        assert f(2, 1 << 12, 64, *ins, None, P2, P, 16, None) == WORKSPACE, name
    fc = lib.linrec_scan_complex_normalized
    assert fc(0, 4, 4, None, None, None, None, None, 0, None) == OK
    assert fc(2, 1 << 12, 64, P, None, None, P2, P, needc, None) == INVALID
    assert fc(2, 1 << 12, 64, P, ctypes.c_void_p(0x100004), None, P2, P, needc, None) == UNSUPPORTED
    assert fc(2, 1 << 12, 64, P, P, None, P2, P, 16, None) == WORKSPACE


def test_wkv4_backward_ex_argument_checks(lib):
    f = lib.wkv4_backward_ex
    need = lib.wkv4_backward_workspace_size(2, 1000, 64)

    def call(r=P, s_in=None, s_out=None, gy=P, gs_out=None, gr=P2, gs_in=None, ws=need, T=1000):
        # (B, T, C, w, u, k, v, r, s_in, s_out, gy, gs_out, gw, gu, gk, gv, gr, gs_in, ws, bytes, stream)
        return f(2, T, 64, P, P, P, P, r, s_in, s_out, gy, gs_out, P2, P2, P2, P2, gr, gs_in, P, ws, None)

    # r and gr must come together
    assert call(gr=None) == INVALID
    assert call(r=None) == INVALID
    # alignment of the gate and state pointers
    assert call(r=ODD) == UNSUPPORTED
    assert call(gr=ODD) == UNSUPPORTED
    assert call(s_in=ODD) == UNSUPPORTED
    assert call(gs_in=ODD) == UNSUPPORTED
    assert call(s_out=P, gs_out=ODD) == UNSUPPORTED
    # the final state's gradient needs its exponents
    assert call(gs_out=P2) == INVALID
    assert call(gs_out=P2, T=0) == INVALID
    # workspace, required pointers
    assert call(ws=16) == WORKSPACE
    assert call(gy=None) == INVALID

def test_wkv4_checkpoint_argument_checks(lib):
    B, T, C = 2, 1000, 64
    nck = lib.wkv4_checkpoint_size(B, T, C)
    nfw = lib.wkv4_forward_ckpt_workspace_size(B, T, C)
    nbw = lib.wkv4_backward_ckpt_workspace_size(B, T, C)
    # one record (4 float32 mantissas and their exponent, 20 bytes) per slab of 56 steps,
    # channel and batch row; the backward's workspace drops the state pass
    assert nck == B * C * ((T + 55) // 56) * 20
    assert 0 < nbw < lib.wkv4_backward_workspace_size(B, T, C)
    assert nfw > 0
    assert lib.wkv4_checkpoint_size(0, T, C) == 0 and lib.wkv4_checkpoint_size(-1, T, C) == 0

    def fw(ck=P2, nc=nck, ws=P, nws=nfw, y=P2, k=P, r=None):
        return lib.wkv4_forward_ckpt(B, T, C, P, P, k, P, r, y, ck, nc, ws, nws, None)

    def bw(ck=P2, nc=nck, ws=P, nws=nbw, gy=P, gw=P2, r=None, gr=None):
        return lib.wkv4_backward_ckpt(B, T, C, P, P, P, P, r, gy, ck, nc, gw, P2, P2, P2, gr, ws, nws, None)

    for f in (fw, bw):
        assert f(nc=nck - 1) == WORKSPACE
        assert b"checkpoint" in lib.linrec_last_error()
        assert f(ck=None) == INVALID
        assert f(ck=ctypes.c_void_p(0x200008)) == UNSUPPORTED
        assert f(nws=16) == WORKSPACE
        assert f(ws=None) == INVALID
    assert fw(y=None) == INVALID
    assert fw(k=ODD) == UNSUPPORTED
    assert fw(r=ODD) == UNSUPPORTED
    assert bw(gy=None) == INVALID
    assert bw(gw=None) == INVALID
    # the gate and its gradient come together
    assert bw(r=P) == INVALID
    assert bw(gr=P) == INVALID
    assert bw(r=ODD, gr=P) == UNSUPPORTED
    assert lib.wkv4_forward_ckpt(-1, T, C, P, P, P, P, None, P2, P2, nck, P, nfw, None) == INVALID
    # empty shapes return before any launch: nothing to do (B = 0), nothing read
    assert lib.wkv4_forward_ckpt(0, T, C, None, None, None, None, None, None, None, 0, None, 0, None) == OK
    assert lib.wkv4_backward_ckpt(B, T, 0, None, None, None, None, None, None, None, 0, None, None, None, None,
                                  None, None, 0, None) == OK


def test_noalloc_forward_host_checks(lib):
    """wkv4_forward_noalloc: the same argument checks as wkv4_forward, and a launch that would
    need more scratch than the library's static array holds is refused before any HIP call."""
    m = re.search(r"#define LINREC_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", open(HEADER).read())
    limit = int(m.group(1)) << 20
    na = lib.wkv4_forward_noalloc
    assert na(-1, 4, 4, P, P, P, P, P2, None) == INVALID
    assert na(1, 4, 4, P, None, P, P, P2, None) == INVALID
    assert na(1, 4, 4, P, P, ODD, P, P2, None) == UNSUPPORTED
    assert na(0, 16, 16, P, P, P, P, P2, None) == OK
    assert na(2, 0, 16, None, None, None, None, None, None) == OK
    # The bench and long-context shapes fit; a much larger one does not.
    assert lib.wkv4_forward_workspace_size(8, 1024, 768) < limit
    assert lib.wkv4_forward_workspace_size(64, 65536, 1024) > limit
    assert na(64, 65536, 1024, P, P, P, P, P2, None) == UNSUPPORTED
    assert b"scratch" in lib.linrec_last_error()
