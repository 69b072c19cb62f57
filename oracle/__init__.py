"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may import
this package.  The HIP library and its Python binding never import, link or call it, and
it imports nothing from them.

``oracle.c`` holds the plain C reference (see the comments there for the passages each
routine follows); this module compiles it with gcc (``-O2 -fopenmp``, no fast-math) into
``liboracle.so`` next to it and wraps it with ctypes.  Inputs are float32 / complex64
numpy arrays, exactly the arrays handed to the GPU; outputs are float64 / complex128.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc, -O2, OpenMP, IEEE double)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_wkv4_forward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_wkv4_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P,
                                         _F32P, _F64P, _F64P, _F64P, _F64P]
    lib.oracle_scan_real.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_scan_complex.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_wkv4_forward_ex.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P, _F32P, _F32P,
                                           _F64P, _F64P]
    lib.oracle_wkv4_forward_ex.restype = None
    lib.oracle_scan_real_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F64P, _F32P,
                                              _F64P, _F64P, _F64P]
    lib.oracle_scan_complex_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F64P, _F32P,
                                                 _F64P, _F64P, _F64P]
    lib.oracle_token_shift.argtypes = [_I64, _I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_token_shift_backward.argtypes = [_I64, _I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P,
                                                _F64P, _F64P, _F64P]
    lib.oracle_wkv4_backward_gated.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P, _F32P, _F32P,
                                               _F64P, _F64P, _F64P, _F64P, _F64P]
    lib.oracle_wkv4_backward_gated.restype = None
    lib.oracle_wkv4_backward_ex.argtypes = [_I64, _I64, _I64] + [_F32P] * 9 + [_F64P] * 6
    lib.oracle_wkv4_backward_ex.restype = None
    lib.oracle_wkv4_backward_cond.argtypes = [_I64, _I64, _I64] + [_F32P] * 9 + [_F64P] * 8
    lib.oracle_wkv4_backward_cond.restype = None
    lib.oracle_scan_mingru.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_scan_minlstm.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_scan_real_decay.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_scan_complex_normalized.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P]
    lib.oracle_scan_mingru_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P, _F32P,
                                                _F64P, _F64P, _F64P]
    lib.oracle_scan_minlstm_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F32P, _F64P, _F32P,
                                                 _F64P, _F64P, _F64P, _F64P]
    lib.oracle_scan_real_decay_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F64P, _F32P,
                                                    _F64P, _F64P, _F64P]
    lib.oracle_scan_complex_normalized_backward.argtypes = [_I64, _I64, _I64, _F32P, _F32P, _F32P, _F64P, _F32P,
                                                            _F64P, _F64P, _F64P]
    for name in ("oracle_scan_mingru", "oracle_scan_minlstm", "oracle_scan_real_decay",
                 "oracle_scan_complex_normalized", "oracle_scan_mingru_backward", "oracle_scan_minlstm_backward",
                 "oracle_scan_real_decay_backward", "oracle_scan_complex_normalized_backward"):
        getattr(lib, name).restype = None
    for name in ("oracle_wkv4_forward", "oracle_wkv4_backward", "oracle_scan_real",
                 "oracle_scan_complex", "oracle_scan_real_backward", "oracle_scan_complex_backward",
                 "oracle_token_shift", "oracle_token_shift_backward"):
        getattr(lib, name).restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = _bind(_LIB_PATH)
    return _lib


def compile_variant(src_text: str, out_path: str):
    """Compile C source text with the same flags into ``out_path`` and bind it.

    Used by the tests that plant mistakes in a copy of ``oracle.c`` to show that the
    pins catch them; the library built from ``oracle.c`` itself is never touched.
    """
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-w", "-o", out_path, c_path, "-lm"]
    subprocess.run(cmd, check=True)
    return _bind(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def num_threads() -> int:
    """OpenMP threads the oracle uses (``OMP_NUM_THREADS`` or all cores)."""
    return int(_load().oracle_num_threads())


def _f32(x, shape=None):
    a = np.ascontiguousarray(x, dtype=np.float32)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _c64f(x, shape):
    a = np.ascontiguousarray(x, dtype=np.complex64)
    if a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a.view(np.float32)


def _p32(a):
    return a.ctypes.data_as(_F32P)


def _p64(a):
    return a.ctypes.data_as(_F64P)


def wkv4_forward(w, u, k, v, lib=None) -> np.ndarray:
    """y (B,T,C) float64 of the WKV-4 operator (RWKV-LLM page, eq. (14))."""
    k = _f32(k)
    B, T, C = k.shape
    v = _f32(v, (B, T, C))
    w = _f32(w, (C,))
    u = _f32(u, (C,))
    y = np.empty((B, T, C), dtype=np.float64)
    (lib or _load()).oracle_wkv4_forward(B, T, C, _p32(w), _p32(u), _p32(k), _p32(v), _p64(y))
    return y


def wkv4_backward(w, u, k, v, gy, lib=None):
    """(gw (C,), gu (C,), gk (B,T,C), gv (B,T,C)) float64: chain rule of eq. (14)."""
    k = _f32(k)
    B, T, C = k.shape
    v = _f32(v, (B, T, C))
    gy = _f32(gy, (B, T, C))
    w = _f32(w, (C,))
    u = _f32(u, (C,))
    gw = np.empty(C, dtype=np.float64)
    gu = np.empty(C, dtype=np.float64)
    gk = np.empty((B, T, C), dtype=np.float64)
    gv = np.empty((B, T, C), dtype=np.float64)
    (lib or _load()).oracle_wkv4_backward(B, T, C, _p32(w), _p32(u), _p32(k), _p32(v), _p32(gy),
                                 _p64(gw), _p64(gu), _p64(gk), _p64(gv))
    return gw, gu, gk, gv


def wkv4_forward_ex(w, u, k, v, r=None, s_in=None, want_state=True, lib=None):
    """(y (B,T,C), s_out (B,C,3) or None) float64: WKV-4 with the receptance gate sigma(r)
    (eq. (15)) and a carried state (a, b, p), A = a e^p, B = b e^p (see oracle.c)."""
    k = _f32(k)
    B, T, C = k.shape
    v = _f32(v, (B, T, C))
    w = _f32(w, (C,))
    u = _f32(u, (C,))
    ra = None if r is None else _f32(r, (B, T, C))
    sa = None if s_in is None else _f32(s_in, (B, C, 3))
    y = np.empty((B, T, C), dtype=np.float64)
    so = np.empty((B, C, 3), dtype=np.float64) if want_state else None
    (lib or _load()).oracle_wkv4_forward_ex(B, T, C, _p32(w), _p32(u), _p32(k), _p32(v),
                                            None if ra is None else _p32(ra), None if sa is None else _p32(sa),
                                            _p64(y), None if so is None else _p64(so))
    return y, so


def scan_real(a, b, x0=None, lib=None) -> np.ndarray:
    """x (B,T,C) float64 of x_t = a_t x_{t-1} + b_t, x_{-1} = x0 (or 0)."""
    a = _f32(a)
    B, T, C = a.shape
    b = _f32(b, (B, T, C))
    x0a = None if x0 is None else _f32(x0, (B, C))
    x = np.empty((B, T, C), dtype=np.float64)
    (lib or _load()).oracle_scan_real(B, T, C, _p32(a), _p32(b),
                             None if x0a is None else _p32(x0a), _p64(x))
    return x


def scan_complex(lam, u, x0=None, lib=None) -> np.ndarray:
    """x (B,T,C) complex128 of x_t = lam x_{t-1} + u_t, x_{-1} = x0 (or 0)."""
    u = np.ascontiguousarray(u, dtype=np.complex64)
    B, T, C = u.shape
    lf = _c64f(lam, (C,))
    uf = u.view(np.float32)
    x0f = None if x0 is None else _c64f(x0, (B, C))
    x = np.empty((B, T, C), dtype=np.complex128)
    (lib or _load()).oracle_scan_complex(B, T, C, _p32(lf), _p32(uf),
                                None if x0f is None else _p32(x0f),
                                x.view(np.float64).ctypes.data_as(_F64P))
    return x


def scan_real_backward(a, x, gx, x0=None, want_gx0=None, lib=None):
    """(ga, gb (B,T,C), gx0 (B,C) or None) float64: the adjoint of x_t = a_t x_{t-1} + b_t
    for upstream gradients gx, given the forward output x (float32 or float64).  gx0 is
    returned when ``want_gx0`` (default: when x0 is given)."""
    a = _f32(a)
    B, T, C = a.shape
    gx = _f32(gx, (B, T, C))
    xd = np.ascontiguousarray(x, dtype=np.float64)
    if xd.shape != (B, T, C):
        raise ValueError("x must be (B,T,C)")
    x0a = None if x0 is None else _f32(x0, (B, C))
    ga = np.empty((B, T, C), dtype=np.float64)
    gb = np.empty((B, T, C), dtype=np.float64)
    gx0 = np.empty((B, C), dtype=np.float64) if (x0 is not None if want_gx0 is None else want_gx0) else None
    (lib or _load()).oracle_scan_real_backward(B, T, C, _p32(a), None if x0a is None else _p32(x0a),
                                               _p64(xd), _p32(gx), _p64(ga), _p64(gb),
                                               None if gx0 is None else _p64(gx0))
    return ga, gb, gx0


def scan_complex_backward(lam, x, gx, x0=None, want_gx0=None, lib=None):
    """(glam (C,), gu (B,T,C), gx0 (B,C) or None) complex128: the adjoint of
    x_t = lam x_{t-1} + u_t (gradients as dL/dRe + i dL/dIm), given the forward output x."""
    gxc = np.ascontiguousarray(gx, dtype=np.complex64)
    B, T, C = gxc.shape
    lf = _c64f(lam, (C,))
    xd = np.ascontiguousarray(x, dtype=np.complex128)
    if xd.shape != (B, T, C):
        raise ValueError("x must be (B,T,C)")
    x0f = None if x0 is None else _c64f(x0, (B, C))
    glam = np.empty(C, dtype=np.complex128)
    gu = np.empty((B, T, C), dtype=np.complex128)
    gx0 = np.empty((B, C), dtype=np.complex128) if (x0 is not None if want_gx0 is None else want_gx0) else None
    f64 = lambda z: z.view(np.float64).ctypes.data_as(_F64P)  # noqa: E731
    (lib or _load()).oracle_scan_complex_backward(B, T, C, _p32(lf), None if x0f is None else _p32(x0f),
                                                  f64(xd), _p32(gxc.view(np.float32)), f64(glam), f64(gu),
                                                  None if gx0 is None else f64(gx0))
    return glam, gu, gx0


def token_shift(x, mu, x_prev=None, lib=None) -> np.ndarray:
    """(M,B,T,C) float64: mu[m] x_t + (1 - mu[m]) x_{t-1}, x_{-1} = x_prev or 0 (RWKV-LLM page,
    eqs. (11)-(13))."""
    x = _f32(x)
    B, T, C = x.shape
    mu = _f32(mu)
    M = mu.shape[0]
    mu = _f32(mu, (M, C))
    xp = None if x_prev is None else _f32(x_prev, (B, C))
    out = np.empty((M, B, T, C), dtype=np.float64)
    (lib or _load()).oracle_token_shift(B, T, C, M, _p32(x), None if xp is None else _p32(xp), _p32(mu), _p64(out))
    return out


def token_shift_backward(x, mu, g, x_prev=None, want_gx_prev=True, lib=None):
    """(gx (B,T,C), gmu (M,C), gx_prev (B,C) or None) float64 of token_shift given g = dL/dout."""
    x = _f32(x)
    B, T, C = x.shape
    mu = _f32(mu)
    M = mu.shape[0]
    mu = _f32(mu, (M, C))
    g = _f32(g, (M, B, T, C))
    xp = None if x_prev is None else _f32(x_prev, (B, C))
    gx = np.empty((B, T, C), dtype=np.float64)
    gmu = np.empty((M, C), dtype=np.float64)
    gxp = np.empty((B, C), dtype=np.float64) if want_gx_prev else None
    (lib or _load()).oracle_token_shift_backward(B, T, C, M, _p32(x), None if xp is None else _p32(xp), _p32(mu),
                                                 _p32(g), _p64(gx), _p64(gmu), None if gxp is None else _p64(gxp))
    return gx, gmu, gxp


def scan_mingru(kz, h, x0=None, lib=None) -> np.ndarray:
    """x (B,T,C) float64 of minGRU: z = sigmoid(kz), x_t = (1 - z_t) x_{t-1} + z_t h_t."""
    kz = _f32(kz)
    B, T, C = kz.shape
    h = _f32(h, (B, T, C))
    x0a = None if x0 is None else _f32(x0, (B, C))
    x = np.empty((B, T, C), dtype=np.float64)
    (lib or _load()).oracle_scan_mingru(B, T, C, _p32(kz), _p32(h), None if x0a is None else _p32(x0a), _p64(x))
    return x


def scan_minlstm(kf, ki, h, x0=None, lib=None) -> np.ndarray:
    """x (B,T,C) float64 of minLSTM: f, i = sigmoid(kf), sigmoid(ki), normalised to sum to 1."""
    kf = _f32(kf)
    B, T, C = kf.shape
    ki = _f32(ki, (B, T, C))
    h = _f32(h, (B, T, C))
    x0a = None if x0 is None else _f32(x0, (B, C))
    x = np.empty((B, T, C), dtype=np.float64)
    (lib or _load()).oracle_scan_minlstm(B, T, C, _p32(kf), _p32(ki), _p32(h),
                                         None if x0a is None else _p32(x0a), _p64(x))
    return x


def scan_real_decay(lam, u, x0=None, lib=None) -> np.ndarray:
    """x (B,T,C) float64 of x_t = lam_c x_{t-1} + u_t (lam (C,))."""
    u = _f32(u)
    B, T, C = u.shape
    lam = _f32(lam, (C,))
    x0a = None if x0 is None else _f32(x0, (B, C))
    x = np.empty((B, T, C), dtype=np.float64)
    (lib or _load()).oracle_scan_real_decay(B, T, C, _p32(lam), _p32(u), None if x0a is None else _p32(x0a), _p64(x))
    return x


def scan_complex_normalized(lam, u, x0=None, lib=None) -> np.ndarray:
    """x (B,T,C) complex128 of x_t = lam x_{t-1} + sqrt(1 - |lam|^2) u_t."""
    u = np.ascontiguousarray(u, dtype=np.complex64)
    B, T, C = u.shape
    lamf = _c64f(lam, (C,))
    uf = u.view(np.float32)
    x0f = None if x0 is None else _c64f(x0, (B, C))
    x = np.empty((B, T, C), dtype=np.complex128)
    (lib or _load()).oracle_scan_complex_normalized(B, T, C, _p32(lamf), _p32(uf), None if x0f is None else _p32(x0f),
                                                    x.view(np.float64).ctypes.data_as(_F64P))
    return x


def _want(x0, want_gx0):
    return x0 is not None if want_gx0 is None else want_gx0


def _x64(x, shape):
    xd = np.ascontiguousarray(x, dtype=np.float64)
    if xd.shape != shape:
        raise ValueError("x must be %s" % (shape,))
    return xd


def scan_mingru_backward(kz, h, x, gx, x0=None, want_gx0=None, lib=None):
    """(gkz, gh (B,T,C), gx0 (B,C) or None) float64: the backward of minGRU given its forward
    output x and the upstream gradient gx."""
    kz = _f32(kz)
    B, T, C = kz.shape
    h, gx = _f32(h, (B, T, C)), _f32(gx, (B, T, C))
    xd = _x64(x, (B, T, C))
    x0a = None if x0 is None else _f32(x0, (B, C))
    gkz, gh = np.empty((B, T, C)), np.empty((B, T, C))
    gx0 = np.empty((B, C)) if _want(x0, want_gx0) else None
    (lib or _load()).oracle_scan_mingru_backward(B, T, C, _p32(kz), _p32(h), None if x0a is None else _p32(x0a),
                                                 _p64(xd), _p32(gx), _p64(gkz), _p64(gh),
                                                 None if gx0 is None else _p64(gx0))
    return gkz, gh, gx0


def scan_minlstm_backward(kf, ki, h, x, gx, x0=None, want_gx0=None, lib=None):
    """(gkf, gki, gh (B,T,C), gx0 (B,C) or None) float64: the backward of minLSTM."""
    kf = _f32(kf)
    B, T, C = kf.shape
    ki, h, gx = _f32(ki, (B, T, C)), _f32(h, (B, T, C)), _f32(gx, (B, T, C))
    xd = _x64(x, (B, T, C))
    x0a = None if x0 is None else _f32(x0, (B, C))
    gkf, gki, gh = np.empty((B, T, C)), np.empty((B, T, C)), np.empty((B, T, C))
    gx0 = np.empty((B, C)) if _want(x0, want_gx0) else None
    (lib or _load()).oracle_scan_minlstm_backward(B, T, C, _p32(kf), _p32(ki), _p32(h),
                                                  None if x0a is None else _p32(x0a), _p64(xd), _p32(gx),
                                                  _p64(gkf), _p64(gki), _p64(gh), None if gx0 is None else _p64(gx0))
    return gkf, gki, gh, gx0


def scan_real_decay_backward(lam, x, gx, x0=None, want_gx0=None, lib=None):
    """(glam (C,), gu (B,T,C), gx0 (B,C) or None) float64: the backward of
    x_t = lam_c x_{t-1} + u_t."""
    gx = _f32(gx)
    B, T, C = gx.shape
    lam = _f32(lam, (C,))
    xd = _x64(x, (B, T, C))
    x0a = None if x0 is None else _f32(x0, (B, C))
    glam, gu = np.empty(C), np.empty((B, T, C))
    gx0 = np.empty((B, C)) if _want(x0, want_gx0) else None
    (lib or _load()).oracle_scan_real_decay_backward(B, T, C, _p32(lam), None if x0a is None else _p32(x0a),
                                                     _p64(xd), _p32(gx), _p64(glam), _p64(gu),
                                                     None if gx0 is None else _p64(gx0))
    return glam, gu, gx0


def scan_complex_normalized_backward(lam, u, x, gx, x0=None, want_gx0=None, lib=None):
    """(glam (C,), gu (B,T,C), gx0 (B,C) or None) complex128: the backward of
    x_t = lam x_{t-1} + sqrt(1 - |lam|^2) u_t (gradients as dL/dRe + i dL/dIm)."""
    gxc = np.ascontiguousarray(gx, dtype=np.complex64)
    B, T, C = gxc.shape
    lf = _c64f(lam, (C,))
    uc = np.ascontiguousarray(u, dtype=np.complex64)
    if uc.shape != (B, T, C):
        raise ValueError("u must be (B,T,C)")
    xd = np.ascontiguousarray(x, dtype=np.complex128)
    if xd.shape != (B, T, C):
        raise ValueError("x must be (B,T,C)")
    x0f = None if x0 is None else _c64f(x0, (B, C))
    glam = np.empty(C, dtype=np.complex128)
    gu = np.empty((B, T, C), dtype=np.complex128)
    gx0 = np.empty((B, C), dtype=np.complex128) if _want(x0, want_gx0) else None
    f64 = lambda z: z.view(np.float64).ctypes.data_as(_F64P)  # noqa: E731
    (lib or _load()).oracle_scan_complex_normalized_backward(
        B, T, C, _p32(lf), _p32(uc.view(np.float32)), None if x0f is None else _p32(x0f), f64(xd),
        _p32(gxc.view(np.float32)), f64(glam), f64(gu), None if gx0 is None else f64(gx0))
    return glam, gu, gx0


def wkv4_backward_gated(w, u, k, v, r, gy, lib=None):
    """(gw, gu, gk, gv, gr) float64 of the gated output sigma(r) wkv (eq. (15)) given gy."""
    k = _f32(k)
    B, T, C = k.shape
    v, r, gy = _f32(v, (B, T, C)), _f32(r, (B, T, C)), _f32(gy, (B, T, C))
    w, u = _f32(w, (C,)), _f32(u, (C,))
    gw, gu = np.empty(C), np.empty(C)
    gk, gv, gr = (np.empty((B, T, C)) for _ in range(3))
    (lib or _load()).oracle_wkv4_backward_gated(B, T, C, _p32(w), _p32(u), _p32(k), _p32(v), _p32(r), _p32(gy),
                                                _p64(gw), _p64(gu), _p64(gk), _p64(gv), _p64(gr))
    return gw, gu, gk, gv, gr


def wkv4_backward_ex(w, u, k, v, gy, r=None, s_in=None, s_out=None, gs_out=None, want_gs_in=True, lib=None):
    """(gw, gu, gk, gv, gr or None, gs_in (B,C,2) or None) float64 of WKV-4 with the optional
    gate sigma(r) and carried state: s_in (a, b, p); gs_out = dL/d(a', b') of s_out = (a', b', p')
    (p' fixed); gs_in = dL/d(a, b) of s_in (its p fixed)."""
    k = _f32(k)
    B, T, C = k.shape
    v, gy = _f32(v, (B, T, C)), _f32(gy, (B, T, C))
    w, u = _f32(w, (C,)), _f32(u, (C,))
    ra = None if r is None else _f32(r, (B, T, C))
    si = None if s_in is None else _f32(s_in, (B, C, 3))
    so = None if s_out is None else _f32(s_out, (B, C, 3))
    go = None if gs_out is None else _f32(gs_out, (B, C, 2))
    gw, gu = np.empty(C), np.empty(C)
    gk, gv = np.empty((B, T, C)), np.empty((B, T, C))
    gr = None if ra is None else np.empty((B, T, C))
    gsi = np.empty((B, C, 2)) if want_gs_in else None
    opt = lambda a, f: None if a is None else f(a)  # noqa: E731
    (lib or _load()).oracle_wkv4_backward_ex(B, T, C, _p32(w), _p32(u), _p32(k), _p32(v), opt(ra, _p32), opt(si, _p32),
                                             opt(so, _p32), _p32(gy), opt(go, _p32), _p64(gw), _p64(gu), _p64(gk),
                                             _p64(gv), opt(gr, _p64), opt(gsi, _p64))
    return gw, gu, gk, gv, gr, gsi


def wkv4_backward_cond(w, u, k, v, gy, r=None, s_in=None, s_out=None, gs_out=None, lib=None):
    """wkv4_backward_ex's outputs followed by (cw, cu): per channel, the sums over b and t of
    the magnitudes of the products in each term of dL/dw and dL/du (their conditioning; see
    oracle_wkv4_backward_cond).  gs_in is returned when s_in or gs_out is given."""
    k = _f32(k)
    B, T, C = k.shape
    v, gy = _f32(v, (B, T, C)), _f32(gy, (B, T, C))
    w, u = _f32(w, (C,)), _f32(u, (C,))
    ra = None if r is None else _f32(r, (B, T, C))
    si = None if s_in is None else _f32(s_in, (B, C, 3))
    so = None if s_out is None else _f32(s_out, (B, C, 3))
    go = None if gs_out is None else _f32(gs_out, (B, C, 2))
    gw, gu, cw, cu = np.empty(C), np.empty(C), np.empty(C), np.empty(C)
    gk, gv = np.empty((B, T, C)), np.empty((B, T, C))
    gr = None if ra is None else np.empty((B, T, C))
    gsi = np.empty((B, C, 2)) if (si is not None or go is not None) else None
    opt = lambda a, f: None if a is None else f(a)  # noqa: E731
    (lib or _load()).oracle_wkv4_backward_cond(B, T, C, _p32(w), _p32(u), _p32(k), _p32(v), opt(ra, _p32),
                                               opt(si, _p32), opt(so, _p32), _p32(gy), opt(go, _p32), _p64(gw),
                                               _p64(gu), _p64(gk), _p64(gv), opt(gr, _p64), opt(gsi, _p64),
                                               _p64(cw), _p64(cu))
    return gw, gu, gk, gv, gr, gsi, cw, cu
