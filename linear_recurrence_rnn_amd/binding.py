"""Thin ctypes binding of ``liblinrec.so`` (the C ABI in ``include/linrec.h``).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, a ``LinrecError`` is raised.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch  # imported before the library so both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinrec.so")

LINREC_OK = 0
LINREC_ERR_INVALID_ARG = 1
LINREC_ERR_WORKSPACE = 2
LINREC_ERR_UNSUPPORTED = 3
LINREC_ERR_HIP = 4

_I64 = ctypes.c_int64
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_lock = threading.Lock()
_lib = None


class LinrecError(RuntimeError):
    """A library call returned an error status."""

    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (func, status_string(status), detail))


def load(path: str | None = None):
    """Load the library once (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise LinrecError(-1, "load", "%s is missing; build it with "
                              "`python -m linear_recurrence_rnn_amd.build`" % p)
        lib = ctypes.CDLL(p)
        lib.linrec_abi_version.restype = ctypes.c_int
        lib.linrec_status_string.restype = ctypes.c_char_p
        lib.linrec_status_string.argtypes = [ctypes.c_int]
        lib.linrec_last_error.restype = ctypes.c_char_p
        for name in ("wkv4_forward_workspace_size", "wkv4_backward_workspace_size", "wkv4_checkpoint_size",
                     "wkv4_forward_ckpt_workspace_size", "wkv4_backward_ckpt_workspace_size"):
            getattr(lib, name).restype = _SZ
            getattr(lib, name).argtypes = [_I64, _I64, _I64]
        lib.linrec_scan_workspace_size.restype = _SZ
        lib.linrec_scan_workspace_size.argtypes = [_I64, _I64, _I64, ctypes.c_int]
        lib.wkv4_forward.restype = ctypes.c_int
        lib.wkv4_forward.argtypes = [_I64, _I64, _I64] + [_VP] * 5 + [_VP, _SZ, _VP]
        lib.wkv4_forward_ex.restype = ctypes.c_int
        lib.wkv4_forward_noalloc.restype = ctypes.c_int
        lib.wkv4_forward_noalloc.argtypes = [_I64, _I64, _I64] + [_VP] * 5 + [_VP]
        lib.wkv4_forward_ex.argtypes = [_I64, _I64, _I64] + [_VP] * 8 + [_VP, _SZ, _VP]
        lib.wkv4_backward.restype = ctypes.c_int
        for name, n in (("linrec_scan_mingru", 4), ("linrec_scan_minlstm", 5), ("linrec_scan_real_decay", 4),
                        ("linrec_scan_complex_normalized", 4)):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = [_I64, _I64, _I64] + [_VP] * n + [_VP, _SZ, _VP]
        lib.rwkv_token_shift.restype = ctypes.c_int
        lib.rwkv_token_shift.argtypes = [_I64, _I64, _I64, _I64] + [_VP] * 4 + [_VP]
        lib.rwkv_token_shift_backward_workspace_size.restype = _SZ
        lib.rwkv_token_shift_backward_workspace_size.argtypes = [_I64, _I64, _I64, _I64]
        lib.rwkv_token_shift_backward.restype = ctypes.c_int
        lib.rwkv_token_shift_backward.argtypes = [_I64, _I64, _I64, _I64] + [_VP] * 7 + [_VP, _SZ, _VP]
        lib.wkv4_backward_ex.restype = ctypes.c_int
        lib.wkv4_backward_ex.argtypes = [_I64, _I64, _I64] + [_VP] * 15 + [_VP, _SZ, _VP]
        lib.wkv4_forward_ckpt.restype = ctypes.c_int
        lib.wkv4_forward_ckpt.argtypes = [_I64, _I64, _I64] + [_VP] * 7 + [_SZ, _VP, _SZ, _VP]
        lib.wkv4_backward_ckpt.restype = ctypes.c_int
        lib.wkv4_forward_ckpt_ex.restype = ctypes.c_int
        lib.wkv4_forward_ckpt_ex.argtypes = [_I64, _I64, _I64] + [_VP] * 9 + [_SZ, _VP, _SZ, _VP]
        lib.wkv4_backward_ckpt_ex.restype = ctypes.c_int
        lib.wkv4_backward_ckpt_ex.argtypes = ([_I64, _I64, _I64] + [_VP] * 9 + [_VP, _SZ] + [_VP] * 6 +
                                              [_VP, _SZ, _VP])
        lib.wkv4_backward_ckpt.argtypes = [_I64, _I64, _I64] + [_VP] * 7 + [_SZ] + [_VP] * 5 + [_VP, _SZ, _VP]
        lib.wkv4_decode_step.restype = ctypes.c_int
        lib.wkv4_decode_step.argtypes = [_I64, _I64] + [_VP] * 7 + [_VP]
        lib.wkv4_backward.argtypes = [_I64, _I64, _I64] + [_VP] * 9 + [_VP, _SZ, _VP]
        lib.linrec_scan_real.restype = ctypes.c_int
        lib.linrec_scan_real.argtypes = [_I64, _I64, _I64] + [_VP] * 4 + [_VP, _SZ, _VP]
        lib.linrec_scan_complex.restype = ctypes.c_int
        lib.linrec_scan_complex.argtypes = [_I64, _I64, _I64] + [_VP] * 4 + [_VP, _SZ, _VP]
        lib.linrec_scan_backward_workspace_size.restype = _SZ
        lib.linrec_scan_backward_workspace_size.argtypes = [_I64, _I64, _I64, ctypes.c_int]
        for name, n in (("linrec_scan_real_backward", 7), ("linrec_scan_complex_backward", 7),
                        ("linrec_scan_mingru_backward", 8), ("linrec_scan_minlstm_backward", 10),
                        ("linrec_scan_real_decay_backward", 7), ("linrec_scan_complex_normalized_backward", 8)):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = [_I64, _I64, _I64] + [_VP] * n + [_VP, _SZ, _VP]
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load().linrec_status_string(status).decode()
    except Exception:  # library not loadable: still describe the code
        return str(status)


def _check(status: int, func: str) -> None:
    if status != LINREC_OK:
        raise LinrecError(status, func, load().linrec_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _expect(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d bytes" % (
                workspace.numel() * workspace.element_size(), nbytes))
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def workspace_size(op: str, B: int, T: int, C: int) -> int:
    """Bytes of workspace ``op`` needs ('wkv4_forward', 'wkv4_backward', 'scan_real', 'scan_complex',
    'scan_real_backward', 'scan_complex_backward')."""
    lib = load()
    if op == "wkv4_forward":
        return int(lib.wkv4_forward_workspace_size(B, T, C))
    if op == "wkv4_backward":
        return int(lib.wkv4_backward_workspace_size(B, T, C))
    if op == "scan_real":
        return int(lib.linrec_scan_workspace_size(B, T, C, 0))
    if op == "scan_complex":
        return int(lib.linrec_scan_workspace_size(B, T, C, 1))
    if op == "scan_real_backward":
        return int(lib.linrec_scan_backward_workspace_size(B, T, C, 0))
    if op == "scan_complex_backward":
        return int(lib.linrec_scan_backward_workspace_size(B, T, C, 1))
    raise KeyError(op)


def wkv4_forward(w, u, k, v, out=None, workspace=None):
    """y = WKV-4(w, u, k, v): k, v (B,T,C) float32 on a ROCm device, w, u (C,)."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    _expect(k, "k", torch.float32, (B, T, C), dev)
    _expect(v, "v", torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    y = torch.empty_like(k) if out is None else out
    _expect(y, "out", torch.float32, (B, T, C), dev)
    ws, nws = _workspace(int(lib.wkv4_forward_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_forward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y), _ptr(ws), nws,
                            _stream(dev)), "wkv4_forward")
    return y


def wkv4_forward_noalloc(w, u, k, v, out=None):
    """y as wkv4_forward, through the entry point that takes no workspace (its scratch is a
    static device array of the library; see include/linrec.h for the size limit and the rule
    that calls overlapping on one GPU race)."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    _expect(k, "k", torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    _expect(v, "v", torch.float32, (B, T, C), dev)
    y = out if out is not None else torch.empty_like(k)
    _expect(y, "out", torch.float32, (B, T, C), dev)
    _check(lib.wkv4_forward_noalloc(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y), _stream(dev)),
           "wkv4_forward_noalloc")
    return y


def wkv4_forward_ex(w, u, k, v, r=None, state=None, want_state=True, out=None, workspace=None):
    """(y, state_out) of WKV-4 with the receptance gate sigma(r) and a carried state
    (a, b, p) per (batch row, channel): ``state`` (B,C,3) float32 or None (empty);
    state_out (B,C,3) when ``want_state``."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    _expect(k, "k", torch.float32, (B, T, C), dev)
    _expect(v, "v", torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, T, C), dev)
    if state is not None:
        _expect(state, "state", torch.float32, (B, C, 3), dev)
    if out is None:
        y = torch.empty_like(k)
        s_out = torch.empty((B, C, 3), dtype=torch.float32, device=dev) if want_state else None
    else:
        y, s_out = out
        _expect(y, "out[0]", torch.float32, (B, T, C), dev)
        if s_out is not None:
            _expect(s_out, "out[1]", torch.float32, (B, C, 3), dev)
    ws, nws = _workspace(int(lib.wkv4_forward_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_forward_ex(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(state), _ptr(y),
                               _ptr(s_out), _ptr(ws), nws, _stream(dev)), "wkv4_forward_ex")
    return y, s_out


def wkv4_decode_step(w, u, k, v, state, r=None, out=None):
    """One token of WKV-4 in recurrent form: k, v, r (B,C) float32, ``state`` (B,C,3)
    float32 (a, b, p), updated IN PLACE.  Returns y (B,C)."""
    lib = load()
    B, C = k.shape
    dev = k.device
    _expect(k, "k", torch.float32, (B, C), dev)
    _expect(v, "v", torch.float32, (B, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    _expect(state, "state", torch.float32, (B, C, 3), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, C), dev)
    y = torch.empty_like(k) if out is None else out
    _expect(y, "out", torch.float32, (B, C), dev)
    _check(lib.wkv4_decode_step(B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(state), _ptr(y),
                                _stream(dev)), "wkv4_decode_step")
    return y


def token_shift(x, mu, x_prev=None, out=None):
    """(M,B,T,C) mixes mu[m] x_t + (1 - mu[m]) x_{t-1} of x (B,T,C) float32, mu (M,C);
    x_{-1} = x_prev (B,C) or 0."""
    lib = load()
    B, T, C = x.shape
    dev = x.device
    M = mu.shape[0] if mu.dim() == 2 else -1
    _expect(x, "x", torch.float32, (B, T, C), dev)
    _expect(mu, "mu", torch.float32, (M, C), dev)
    if x_prev is not None:
        _expect(x_prev, "x_prev", torch.float32, (B, C), dev)
    o = torch.empty((M, B, T, C), dtype=torch.float32, device=dev) if out is None else out
    _expect(o, "out", torch.float32, (M, B, T, C), dev)
    _check(lib.rwkv_token_shift(B, T, C, M, _ptr(x), _ptr(x_prev), _ptr(mu), _ptr(o), _stream(dev)),
           "rwkv_token_shift")
    return o


def token_shift_backward(x, mu, g, x_prev=None, want_gx_prev=None, out=None, workspace=None):
    """(gx (B,T,C), gmu (M,C), gx_prev (B,C) or None) of token_shift given g = dL/dout (M,B,T,C).
    gx_prev is returned when ``want_gx_prev`` (default: when x_prev is given)."""
    lib = load()
    B, T, C = x.shape
    dev = x.device
    M = mu.shape[0] if mu.dim() == 2 else -1
    _expect(x, "x", torch.float32, (B, T, C), dev)
    _expect(mu, "mu", torch.float32, (M, C), dev)
    _expect(g, "g", torch.float32, (M, B, T, C), dev)
    if x_prev is not None:
        _expect(x_prev, "x_prev", torch.float32, (B, C), dev)
    if want_gx_prev is None:
        want_gx_prev = x_prev is not None
    if out is None:
        gx = torch.empty_like(x)
        gmu = torch.empty((M, C), dtype=torch.float32, device=dev)
        gxp = torch.empty((B, C), dtype=torch.float32, device=dev) if want_gx_prev else None
    else:
        gx, gmu, gxp = out
    ws, nws = _workspace(int(lib.rwkv_token_shift_backward_workspace_size(B, T, C, M)), dev, workspace)
    _check(lib.rwkv_token_shift_backward(B, T, C, M, _ptr(x), _ptr(x_prev), _ptr(mu), _ptr(g), _ptr(gx), _ptr(gmu),
                                         _ptr(gxp), _ptr(ws), nws, _stream(dev)), "rwkv_token_shift_backward")
    return gx, gmu, gxp


def wkv4_backward_ex(w, u, k, v, gy, r=None, s_in=None, s_out=None, gs_out=None, want_gs_in=True, out=None,
                     workspace=None):
    """(gw, gu, gk, gv, gr, gs_in) of wkv4_forward_ex: gy = dL/d(output); r the gate (gr None
    without it); s_in the carried state (a, b, p) given to the forward or None; s_out the
    forward's final state, read (its p) only with gs_out = dL/d(a', b') (B,C,2); gs_in =
    dL/d(a, b) of s_in (B,C,2) when ``want_gs_in``, else None."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    for name, t in (("k", k), ("v", v), ("gy", gy)):
        _expect(t, name, torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, T, C), dev)
    for name, t, n in (("s_in", s_in, 3), ("s_out", s_out, 3), ("gs_out", gs_out, 2)):
        if t is not None:
            _expect(t, name, torch.float32, (B, C, n), dev)
    if gs_out is not None and s_out is None:
        raise ValueError("gs_out needs s_out (the forward's final state)")
    if out is None:
        gw, gu = torch.empty_like(w), torch.empty_like(u)
        gk, gv = torch.empty_like(k), torch.empty_like(k)
        gr = None if r is None else torch.empty_like(k)
        gs_in = torch.empty((B, C, 2), dtype=torch.float32, device=dev) if want_gs_in else None
    else:
        gw, gu, gk, gv, gr, gs_in = out
        for name, t, shape in (("gw", gw, (C,)), ("gu", gu, (C,)), ("gk", gk, (B, T, C)), ("gv", gv, (B, T, C))):
            _expect(t, "out " + name, torch.float32, shape, dev)
        if (gr is None) != (r is None):
            raise ValueError("out gr must be given exactly when r is")
        if gr is not None:
            _expect(gr, "out gr", torch.float32, (B, T, C), dev)
        if gs_in is not None:
            _expect(gs_in, "out gs_in", torch.float32, (B, C, 2), dev)
    ws, nws = _workspace(int(lib.wkv4_backward_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_backward_ex(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(s_in), _ptr(s_out),
                                _ptr(gy), _ptr(gs_out), _ptr(gw), _ptr(gu), _ptr(gk), _ptr(gv), _ptr(gr),
                                _ptr(gs_in), _ptr(ws), nws, _stream(dev)), "wkv4_backward_ex")
    return gw, gu, gk, gv, gr, gs_in


def wkv4_backward_gated(w, u, k, v, r, gy, out=None, workspace=None):
    """(gw, gu, gk, gv, gr) of the gated output sigma(r) wkv given gy = dL/d(output)."""
    _expect(r, "r", torch.float32, tuple(k.shape), k.device)
    return wkv4_backward_ex(w, u, k, v, gy, r=r, want_gs_in=False,
                            out=None if out is None else tuple(out) + (None,), workspace=workspace)[:5]


def wkv4_backward(w, u, k, v, gy, out=None, workspace=None):
    """(gw, gu, gk, gv) = gradients of sum(gy * WKV-4(w, u, k, v))."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    for name, t in (("k", k), ("v", v), ("gy", gy)):
        _expect(t, name, torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    if out is None:
        gw = torch.empty(C, dtype=torch.float32, device=dev)
        gu = torch.empty(C, dtype=torch.float32, device=dev)
        gk = torch.empty_like(k)
        gv = torch.empty_like(k)
    else:
        gw, gu, gk, gv = out
    ws, nws = _workspace(int(lib.wkv4_backward_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_backward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(gy), _ptr(gw),
                             _ptr(gu), _ptr(gk), _ptr(gv), _ptr(ws), nws, _stream(dev)),
           "wkv4_backward")
    return gw, gu, gk, gv


def wkv4_checkpoint_size(B: int, T: int, C: int) -> int:
    """Bytes of the checkpoint buffer of wkv4_forward_ckpt / wkv4_backward_ckpt."""
    return int(load().wkv4_checkpoint_size(B, T, C))


def wkv4_forward_ckpt(w, u, k, v, r=None, out=None, workspace=None):
    """(y, ckpt): y as wkv4_forward (gated by sigma(r) when ``r`` is given), and ckpt (uint8
    device buffer) holding the forward sums that wkv4_backward_ckpt starts its slabs from.
    ``out`` = (y, ckpt) to reuse buffers."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    _expect(k, "k", torch.float32, (B, T, C), dev)
    _expect(v, "v", torch.float32, (B, T, C), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    nck = int(lib.wkv4_checkpoint_size(B, T, C))
    if out is None:
        y = torch.empty_like(k)
        ckpt = torch.empty(nck, dtype=torch.uint8, device=dev)
    else:
        y, ckpt = out
        _expect(y, "out[0]", torch.float32, (B, T, C), dev)
        _expect(ckpt, "out[1]", torch.uint8, (nck,), dev)
    ws, nws = _workspace(int(lib.wkv4_forward_ckpt_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_forward_ckpt(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(y), _ptr(ckpt), nck,
                                 _ptr(ws), nws, _stream(dev)), "wkv4_forward_ckpt")
    return y, ckpt


def wkv4_backward_ckpt(w, u, k, v, gy, ckpt, r=None, out=None, workspace=None):
    """(gw, gu, gk, gv) as wkv4_backward, from the ckpt that wkv4_forward_ckpt wrote for the
    same w, u, k, v; with ``r``, the gradients of the gated output sigma(r) wkv and
    (gw, gu, gk, gv, gr)."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    for name, t in (("k", k), ("v", v), ("gy", gy)):
        _expect(t, name, torch.float32, (B, T, C), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, T, C), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    nck = int(lib.wkv4_checkpoint_size(B, T, C))
    _expect(ckpt, "ckpt", torch.uint8, (nck,), dev)
    if out is None:
        gw = torch.empty(C, dtype=torch.float32, device=dev)
        gu = torch.empty(C, dtype=torch.float32, device=dev)
        gk = torch.empty_like(k)
        gv = torch.empty_like(k)
        gr = torch.empty_like(k) if r is not None else None
    else:
        gw, gu, gk, gv = out[:4]
        gr = out[4] if r is not None else None
        _expect(gw, "out[0]", torch.float32, (C,), dev)
        _expect(gu, "out[1]", torch.float32, (C,), dev)
        _expect(gk, "out[2]", torch.float32, (B, T, C), dev)
        _expect(gv, "out[3]", torch.float32, (B, T, C), dev)
        if gr is not None:
            _expect(gr, "out[4]", torch.float32, (B, T, C), dev)
    ws, nws = _workspace(int(lib.wkv4_backward_ckpt_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_backward_ckpt(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(gy), _ptr(ckpt), nck,
                                  _ptr(gw), _ptr(gu), _ptr(gk), _ptr(gv), _ptr(gr), _ptr(ws), nws, _stream(dev)),
           "wkv4_backward_ckpt")
    return (gw, gu, gk, gv) if r is None else (gw, gu, gk, gv, gr)


def wkv4_forward_ckpt_ex(w, u, k, v, r=None, state=None, want_state=True, workspace=None):
    """(y, ckpt, state_out): wkv4_forward_ckpt starting from the carried state ``state``
    (B,C,3) (a, b, p) or None (empty), with the state after the last token (B,C,3) when
    ``want_state``."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    for name, t in (("k", k), ("v", v)):
        _expect(t, name, torch.float32, (B, T, C), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, T, C), dev)
    if state is not None:
        _expect(state, "state", torch.float32, (B, C, 3), dev)
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    nck = int(lib.wkv4_checkpoint_size(B, T, C))
    y = torch.empty_like(k)
    ckpt = torch.empty(max(nck, 1), dtype=torch.uint8, device=dev)
    s_out = torch.empty((B, C, 3), dtype=torch.float32, device=dev) if want_state else None
    ws, nws = _workspace(int(lib.wkv4_forward_ckpt_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_forward_ckpt_ex(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(state), _ptr(y),
                                    _ptr(s_out), _ptr(ckpt), nck, _ptr(ws), nws, _stream(dev)),
           "wkv4_forward_ckpt_ex")
    return y, ckpt, s_out


def wkv4_backward_ckpt_ex(w, u, k, v, gy, ckpt, r=None, s_in=None, s_out=None, gs_out=None, want_gs_in=True,
                          workspace=None):
    """(gw, gu, gk, gv, gr, gs_in) as wkv4_backward_ex, from the ckpt that
    wkv4_forward_ckpt_ex wrote for the same w, u, k, v and s_in (gr None without r, gs_in
    None unless ``want_gs_in``)."""
    lib = load()
    B, T, C = k.shape
    dev = k.device
    for name, t in (("k", k), ("v", v), ("gy", gy)):
        _expect(t, name, torch.float32, (B, T, C), dev)
    if r is not None:
        _expect(r, "r", torch.float32, (B, T, C), dev)
    for name, t, n in (("s_in", s_in, 3), ("s_out", s_out, 3), ("gs_out", gs_out, 2)):
        if t is not None:
            _expect(t, name, torch.float32, (B, C, n), dev)
    if gs_out is not None and s_out is None:
        raise ValueError("gs_out needs s_out (the forward's final state)")
    _expect(w, "w", torch.float32, (C,), dev)
    _expect(u, "u", torch.float32, (C,), dev)
    nck = int(lib.wkv4_checkpoint_size(B, T, C))
    gw, gu = torch.empty_like(w), torch.empty_like(u)
    gk, gv = torch.empty_like(k), torch.empty_like(k)
    gr = None if r is None else torch.empty_like(k)
    gs_in = torch.empty((B, C, 2), dtype=torch.float32, device=dev) if want_gs_in else None
    ws, nws = _workspace(int(lib.wkv4_backward_ckpt_workspace_size(B, T, C)), dev, workspace)
    _check(lib.wkv4_backward_ckpt_ex(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(s_in), _ptr(s_out),
                                     _ptr(gy), _ptr(gs_out), _ptr(ckpt), nck, _ptr(gw), _ptr(gu), _ptr(gk),
                                     _ptr(gv), _ptr(gr), _ptr(gs_in), _ptr(ws), nws, _stream(dev)),
           "wkv4_backward_ckpt_ex")
    return gw, gu, gk, gv, gr, gs_in


def scan_real(a, b, x0=None, out=None, workspace=None):
    """x_t = a_t * x_{t-1} + b_t over (B,T,C) float32; x0 (B,C) or None for zero."""
    lib = load()
    B, T, C = a.shape
    dev = a.device
    _expect(a, "a", torch.float32, (B, T, C), dev)
    _expect(b, "b", torch.float32, (B, T, C), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.float32, (B, C), dev)
    x = torch.empty_like(a) if out is None else out
    _expect(x, "out", torch.float32, (B, T, C), dev)
    ws, nws = _workspace(int(lib.linrec_scan_workspace_size(B, T, C, 0)), dev, workspace)
    _check(lib.linrec_scan_real(B, T, C, _ptr(a), _ptr(b), _ptr(x0), _ptr(x), _ptr(ws), nws,
                                _stream(dev)), "linrec_scan_real")
    return x


def scan_complex(lam, u, x0=None, out=None, workspace=None):
    """x_t = lam * x_{t-1} + u_t over (B,T,C) complex64; lam (C,), x0 (B,C) or None."""
    lib = load()
    B, T, C = u.shape
    dev = u.device
    _expect(u, "u", torch.complex64, (B, T, C), dev)
    _expect(lam, "lam", torch.complex64, (C,), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.complex64, (B, C), dev)
    x = torch.empty_like(u) if out is None else out
    _expect(x, "out", torch.complex64, (B, T, C), dev)
    ws, nws = _workspace(int(lib.linrec_scan_workspace_size(B, T, C, 1)), dev, workspace)
    _check(lib.linrec_scan_complex(B, T, C, _ptr(lam), _ptr(u), _ptr(x0), _ptr(x), _ptr(ws), nws,
                                   _stream(dev)), "linrec_scan_complex")
    return x


def _gated_real(name, tensors, chan, x0, out, workspace):
    lib = load()
    first = tensors[0][1]
    B, T, C = first.shape
    dev = first.device
    for nm, t in tensors:
        _expect(t, nm, torch.float32, (B, T, C), dev)
    if chan is not None:
        _expect(chan, "lam", torch.float32, (C,), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.float32, (B, C), dev)
    x = torch.empty_like(first) if out is None else out
    _expect(x, "out", torch.float32, (B, T, C), dev)
    ws, nws = _workspace(int(lib.linrec_scan_workspace_size(B, T, C, 0)), dev, workspace)
    ptrs = ([_ptr(chan)] if chan is not None else []) + [_ptr(t) for _, t in tensors]
    _check(getattr(lib, name)(B, T, C, *ptrs, _ptr(x0), _ptr(x), _ptr(ws), nws, _stream(dev)), name)
    return x


def scan_mingru(kz, h, x0=None, out=None, workspace=None):
    """minGRU: z = sigmoid(kz), x_t = (1 - z_t) x_{t-1} + z_t h_t; (B,T,C) float32."""
    return _gated_real("linrec_scan_mingru", [("kz", kz), ("h", h)], None, x0, out, workspace)


def scan_minlstm(kf, ki, h, x0=None, out=None, workspace=None):
    """minLSTM: f, i = sigmoid(kf), sigmoid(ki); x_t = (f x_{t-1} + i h_t) / (f + i)."""
    return _gated_real("linrec_scan_minlstm", [("kf", kf), ("ki", ki), ("h", h)], None, x0, out, workspace)


def scan_real_decay(lam, u, x0=None, out=None, workspace=None):
    """x_t = lam_c x_{t-1} + u_t with one decay per channel, lam (C,) float32."""
    return _gated_real("linrec_scan_real_decay", [("u", u)], lam, x0, out, workspace)


def scan_complex_normalized(lam, u, x0=None, out=None, workspace=None):
    """x_t = lam x_{t-1} + sqrt(1 - |lam|^2) u_t over (B,T,C) complex64; lam (C,)."""
    lib = load()
    B, T, C = u.shape
    dev = u.device
    _expect(u, "u", torch.complex64, (B, T, C), dev)
    _expect(lam, "lam", torch.complex64, (C,), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.complex64, (B, C), dev)
    x = torch.empty_like(u) if out is None else out
    _expect(x, "out", torch.complex64, (B, T, C), dev)
    ws, nws = _workspace(int(lib.linrec_scan_workspace_size(B, T, C, 1)), dev, workspace)
    _check(lib.linrec_scan_complex_normalized(B, T, C, _ptr(lam), _ptr(u), _ptr(x0), _ptr(x), _ptr(ws), nws,
                                              _stream(dev)), "linrec_scan_complex_normalized")
    return x


def scan_real_backward(a, x, gx, x0=None, want_gx0=None, out=None, workspace=None):
    """(ga, gb, gx0) = adjoint of x_t = a_t x_{t-1} + b_t for dL/dx = gx, given the forward
    output x.  gx0 is computed when ``want_gx0`` (default: when x0 is given), else None."""
    lib = load()
    B, T, C = a.shape
    dev = a.device
    for name, t in (("a", a), ("x", x), ("gx", gx)):
        _expect(t, name, torch.float32, (B, T, C), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.float32, (B, C), dev)
    if want_gx0 is None:
        want_gx0 = x0 is not None
    if out is None:
        ga, gb = torch.empty_like(a), torch.empty_like(a)
        gx0 = torch.empty((B, C), dtype=torch.float32, device=dev) if want_gx0 else None
    else:
        ga, gb, gx0 = out
    ws, nws = _workspace(int(lib.linrec_scan_backward_workspace_size(B, T, C, 0)), dev, workspace)
    _check(lib.linrec_scan_real_backward(B, T, C, _ptr(a), _ptr(x0), _ptr(x), _ptr(gx), _ptr(ga), _ptr(gb),
                                         _ptr(gx0), _ptr(ws), nws, _stream(dev)), "linrec_scan_real_backward")
    return ga, gb, gx0


def scan_complex_backward(lam, x, gx, x0=None, want_gx0=None, out=None, workspace=None):
    """(glam, gu, gx0) = adjoint of x_t = lam x_{t-1} + u_t for dL/dx = gx (complex
    gradients as dL/dRe + i dL/dIm), given the forward output x."""
    lib = load()
    B, T, C = x.shape
    dev = x.device
    for name, t in (("x", x), ("gx", gx)):
        _expect(t, name, torch.complex64, (B, T, C), dev)
    _expect(lam, "lam", torch.complex64, (C,), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.complex64, (B, C), dev)
    if want_gx0 is None:
        want_gx0 = x0 is not None
    if out is None:
        glam = torch.empty(C, dtype=torch.complex64, device=dev)
        gu = torch.empty_like(x)
        gx0 = torch.empty((B, C), dtype=torch.complex64, device=dev) if want_gx0 else None
    else:
        glam, gu, gx0 = out
    ws, nws = _workspace(int(lib.linrec_scan_backward_workspace_size(B, T, C, 1)), dev, workspace)
    _check(lib.linrec_scan_complex_backward(B, T, C, _ptr(lam), _ptr(x0), _ptr(x), _ptr(gx), _ptr(glam),
                                            _ptr(gu), _ptr(gx0), _ptr(ws), nws, _stream(dev)),
           "linrec_scan_complex_backward")
    return glam, gu, gx0


def _gated_real_backward(name, ins, n_out, chan, x, gx, x0, want_gx0, workspace):
    """Marshals a real variant's adjoint: ``ins`` the (B,T,C) gate/candidate inputs, then x,
    gx; returns the ``n_out`` (B,T,C) gradients, glam (when ``chan`` is given) and gx0."""
    lib = load()
    B, T, C = x.shape
    dev = x.device
    for nm, t in list(ins) + [("x", x), ("gx", gx)]:
        _expect(t, nm, torch.float32, (B, T, C), dev)
    if chan is not None:
        _expect(chan, "lam", torch.float32, (C,), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.float32, (B, C), dev)
    if want_gx0 is None:
        want_gx0 = x0 is not None
    outs = [torch.empty_like(x) for _ in range(n_out)]
    glam = torch.empty(C, dtype=torch.float32, device=dev) if chan is not None else None
    gx0 = torch.empty((B, C), dtype=torch.float32, device=dev) if want_gx0 else None
    ws, nws = _workspace(int(lib.linrec_scan_backward_workspace_size(B, T, C, 0)), dev, workspace)
    if chan is not None:
        ptrs = [_ptr(chan), _ptr(x0), _ptr(x), _ptr(gx), _ptr(glam)] + [_ptr(o) for o in outs]
    else:
        ptrs = [_ptr(t) for _, t in ins] + [_ptr(x0), _ptr(x), _ptr(gx)] + [_ptr(o) for o in outs]
    _check(getattr(lib, name)(B, T, C, *ptrs, _ptr(gx0), _ptr(ws), nws, _stream(dev)), name)
    return tuple(outs) + ((glam,) if chan is not None else ()) + (gx0,)


def scan_mingru_backward(kz, h, x, gx, x0=None, want_gx0=None, workspace=None):
    """(gkz, gh, gx0) of minGRU for dL/dx = gx, given its forward output x."""
    return _gated_real_backward("linrec_scan_mingru_backward", [("kz", kz), ("h", h)], 2, None, x, gx, x0, want_gx0,
                                workspace)


def scan_minlstm_backward(kf, ki, h, x, gx, x0=None, want_gx0=None, workspace=None):
    """(gkf, gki, gh, gx0) of minLSTM for dL/dx = gx, given its forward output x."""
    return _gated_real_backward("linrec_scan_minlstm_backward", [("kf", kf), ("ki", ki), ("h", h)], 3, None, x, gx,
                                x0, want_gx0, workspace)


def scan_real_decay_backward(lam, x, gx, x0=None, want_gx0=None, workspace=None):
    """(glam (C,), gu, gx0) of x_t = lam_c x_{t-1} + u_t for dL/dx = gx, given x."""
    gu, glam, gx0 = _gated_real_backward("linrec_scan_real_decay_backward", [], 1, lam, x, gx, x0, want_gx0,
                                         workspace)
    return glam, gu, gx0


def scan_complex_normalized_backward(lam, u, x, gx, x0=None, want_gx0=None, workspace=None):
    """(glam, gu, gx0) of x_t = lam x_{t-1} + sqrt(1 - |lam|^2) u_t for dL/dx = gx (complex
    gradients as dL/dRe + i dL/dIm), given the input u and the forward output x."""
    lib = load()
    B, T, C = x.shape
    dev = x.device
    for name, t in (("u", u), ("x", x), ("gx", gx)):
        _expect(t, name, torch.complex64, (B, T, C), dev)
    _expect(lam, "lam", torch.complex64, (C,), dev)
    if x0 is not None:
        _expect(x0, "x0", torch.complex64, (B, C), dev)
    if want_gx0 is None:
        want_gx0 = x0 is not None
    glam = torch.empty(C, dtype=torch.complex64, device=dev)
    gu = torch.empty_like(x)
    gx0 = torch.empty((B, C), dtype=torch.complex64, device=dev) if want_gx0 else None
    ws, nws = _workspace(int(lib.linrec_scan_backward_workspace_size(B, T, C, 1)), dev, workspace)
    _check(lib.linrec_scan_complex_normalized_backward(B, T, C, _ptr(lam), _ptr(u), _ptr(x0), _ptr(x), _ptr(gx),
                                                       _ptr(glam), _ptr(gu), _ptr(gx0), _ptr(ws), nws, _stream(dev)),
           "linrec_scan_complex_normalized_backward")
    return glam, gu, gx0
