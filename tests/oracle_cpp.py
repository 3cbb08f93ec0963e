"""ctypes access to the plain C++ statement of the CPU oracle (oracle/cpp/mx_oracle.cpp), built by
__graft_entry__.build() (or here, with g++, when it is missing)."""
import ctypes
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "oracle", "cpp", "libmxoracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_u8 = ctypes.POINTER(ctypes.c_uint8)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(LIB.replace("libmxoracle.so", "mx_oracle.cpp")):
            import sys
            sys.path.insert(0, ROOT)
            import __graft_entry__
            __graft_entry__.build_oracle_cpp()
        L = ctypes.CDLL(LIB)
        L.mxo_e4m3_value.restype = ctypes.c_double
        L.mxo_e4m3_value.argtypes = [ctypes.c_uint8]
        L.mxo_e4m3_code.restype = ctypes.c_uint8
        L.mxo_e4m3_code.argtypes = [ctypes.c_double]
        L.mxo_scale_code.restype = ctypes.c_uint8
        L.mxo_scale_code.argtypes = [ctypes.c_double]
        for f in ("mxo_quantize_row32", "mxo_quantize_col32", "mxo_quantize_sq32"):
            getattr(L, f).restype = None
            getattr(L, f).argtypes = [_d, ctypes.c_int, ctypes.c_int, _u8, _u8]
        L.mxo_attn_fwd.restype = None
        L.mxo_attn_fwd.argtypes = [_d, _d, _d, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int, _d, _d, _u8, _u8]
        L.mxo_attn_bwd.restype = None
        L.mxo_attn_bwd.argtypes = [_d] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int] + [_d] * 4
        _lib = L
    return _lib


def _dp(a):
    return a.ctypes.data_as(_d)


def _up(a):
    return a.ctypes.data_as(_u8)


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, np.float64))


def quantize(layout, x):
    """layout "row32" | "col32" | "sq32" of a 2-D array x [n, d]: (codes [n, d], scales)."""
    x = _f64(x)
    n, d = x.shape
    nb = (n + 31) // 32
    shape = {"row32": (n, d // 32), "col32": (nb, d), "sq32": (nb, (d + 31) // 32)}[layout]
    codes, scales = np.zeros((n, d), np.uint8), np.zeros(shape, np.uint8)
    getattr(lib(), "mxo_quantize_" + layout)(_dp(x), n, d, _up(codes), _up(scales))
    return codes, scales


def attn_fwd(q, k, v, sigma, causal):
    """One head: (O [L, d], LSE [L], P codes [L, L], P scales [L, ceil(L/32)])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, d = q.shape
    O, lse = np.zeros((L, d)), np.zeros(L)
    pc, ps = np.zeros((L, L), np.uint8), np.zeros((L, (L + 31) // 32), np.uint8)
    lib().mxo_attn_fwd(_dp(q), _dp(k), _dp(v), L, d, float(sigma), int(causal), _dp(O), _dp(lse), _up(pc), _up(ps))
    return O, lse, pc, ps


def attn_bwd(q, k, v, o, do, lse, sigma, causal):
    """One head: (dQ, dK, dV [L, d], D [L])."""
    q, k, v, o, do, lse = (_f64(a) for a in (q, k, v, o, do, lse))
    L, d = q.shape
    dq, dk, dv, D = np.zeros((L, d)), np.zeros((L, d)), np.zeros((L, d)), np.zeros(L)
    lib().mxo_attn_bwd(_dp(q), _dp(k), _dp(v), _dp(o), _dp(do), _dp(lse), L, d, float(sigma), int(causal),
                       _dp(dq), _dp(dk), _dp(dv), _dp(D))
    return dq, dk, dv, D
