"""ctypes binding of the fp64 C oracle (oracle.c) — argument marshalling only.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may use it.  Every function takes numpy float32
arrays (the same bytes the GPU path receives), returns float64 results and
raises on a bad argument.  The arithmetic lives entirely in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants a mistake in a copy of oracle.c points this at the copy.
_LIB = os.environ.get("LSE_ORACLE_LIB", _DEFAULT_LIB)
_lib = None

_i64 = ctypes.c_int64
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_DEFAULT_LIB):
        compile_source(_SRC, _DEFAULT_LIB)
    return _DEFAULT_LIB


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load():
    """Load liboracle.so, building it first only if no built copy exists."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            if _LIB != _DEFAULT_LIB:
                raise FileNotFoundError(_LIB)
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_lse_axis0.argtypes = [_f32p, _i64, _i64, _f64p, ctypes.c_int]
        lib.oracle_log_softmax_rows.argtypes = [_f32p, _i64, _i64, _f64p, _f64p,
                                                ctypes.c_int]
        lib.oracle_lse_chunk_partials.argtypes = [_f32p, _i64, _i64, _i64, _f64p,
                                                  _f64p, ctypes.c_int]
        lib.oracle_lse_merge.argtypes = [_f64p, _f64p, _i64, _i64, _f64p, _f64p,
                                         _f64p]
        lib.oracle_hardswish.argtypes = [ctypes.c_double]
        lib.oracle_hardswish.restype = ctypes.c_double
        lib.oracle_conv2d.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _f64p, ctypes.c_int]
        lib.oracle_fused_chain.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _i64,
                                           _i64, _i64, _i64, _i64, _i64, _i64,
                                           ctypes.c_double, _f64p, _f64p, _f64p,
                                           ctypes.c_int]
        lib.oracle_softmax_rows.argtypes = [_f32p, _i64, _i64, _f64p, ctypes.c_int]
        lib.oracle_lse_axis.argtypes = [_f32p, _i64, _i64, _i64, _f64p, ctypes.c_int]
        lib.oracle_log_softmax_axis.argtypes = [_f32p, _i64, _i64, _i64, _f64p, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        for name in ("oracle_lse_axis0", "oracle_log_softmax_rows", "oracle_softmax_rows",
                     "oracle_lse_axis", "oracle_log_softmax_axis",
                     "oracle_lse_chunk_partials", "oracle_lse_merge",
                     "oracle_conv2d", "oracle_fused_chain"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _p32(a):
    return None if a is None else a.ctypes.data_as(_f32p)


def _p64(a):
    return None if a is None else a.ctypes.data_as(_f64p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


def _threads(nthreads):
    return int(nthreads) if nthreads else os.cpu_count() or 1


def max_threads() -> int:
    return int(load().oracle_max_threads())


def lse_axis0(x, nthreads=None) -> np.ndarray:
    """logsumexp over axis 0 of an (R, ...) array; returns shape x.shape[1:]."""
    x = _f32(x)
    R = x.shape[0]
    inner = int(np.prod(x.shape[1:], dtype=np.int64))
    out = np.empty(inner, dtype=np.float64)
    _check(load().oracle_lse_axis0(_p32(x), R, inner, _p64(out), _threads(nthreads)),
           "lse_axis0")
    return out.reshape(x.shape[1:])


def log_softmax_rows(x, want_y=True, nthreads=None):
    """Row-wise log_softmax of a 2-D array -> (y or None, row_lse)."""
    x = _f32(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), dtype=np.float64) if want_y else None
    lse = np.empty(rows, dtype=np.float64)
    _check(load().oracle_log_softmax_rows(_p32(x), rows, cols, _p64(y), _p64(lse),
                                          _threads(nthreads)), "log_softmax_rows")
    return y, lse


def softmax_rows(x, nthreads=None):
    """Row-wise softmax of a 2-D array (float64)."""
    x = _f32(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), dtype=np.float64)
    _check(load().oracle_softmax_rows(_p32(x), rows, cols, _p64(y), _threads(nthreads)),
           "softmax_rows")
    return y


def lse_axis(x, nthreads=None):
    """logsumexp over axis 1 of an (outer, R, inner...) array -> (outer, inner...)."""
    x = _f32(x)
    outer, R = x.shape[0], x.shape[1]
    inner = int(np.prod(x.shape[2:], dtype=np.int64))
    out = np.empty(outer * inner, dtype=np.float64)
    _check(load().oracle_lse_axis(_p32(x), outer, R, inner, _p64(out), _threads(nthreads)),
           "lse_axis")
    return out.reshape((outer,) + x.shape[2:])


def log_softmax_axis(x, nthreads=None):
    """log_softmax over axis 1 of an (outer, R, inner...) array (float64)."""
    x = _f32(x)
    outer, R = x.shape[0], x.shape[1]
    inner = int(np.prod(x.shape[2:], dtype=np.int64))
    y = np.empty(x.shape, dtype=np.float64)
    _check(load().oracle_log_softmax_axis(_p32(x), outer, R, inner, _p64(y),
                                          _threads(nthreads)), "log_softmax_axis")
    return y


def lse_chunk_partials(x, chunk, nthreads=None):
    """(m, s) per (row, chunk) of a 2-D array; each of shape (rows, nchunks)."""
    x = _f32(x)
    rows, cols = x.shape
    k = -(-cols // chunk)
    m = np.empty((rows, k), dtype=np.float64)
    s = np.empty((rows, k), dtype=np.float64)
    _check(load().oracle_lse_chunk_partials(_p32(x), rows, cols, int(chunk), _p64(m),
                                            _p64(s), _threads(nthreads)),
           "lse_chunk_partials")
    return m, s


def lse_merge(m, s):
    """Merge (rows, k) pairs -> (lse, M, S), each of shape (rows,)."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    if m.ndim == 1:
        m, s = m[None, :], s[None, :]
    rows, k = m.shape
    lse = np.empty(rows, dtype=np.float64)
    M = np.empty(rows, dtype=np.float64)
    S = np.empty(rows, dtype=np.float64)
    _check(load().oracle_lse_merge(_p64(m), _p64(s), rows, k, _p64(lse), _p64(M),
                                   _p64(S)), "lse_merge")
    return lse, M, S


def hardswish(t: float) -> float:
    return float(load().oracle_hardswish(float(t)))


def conv2d(x, w, b=None, nthreads=None) -> np.ndarray:
    """Stride-1, unpadded cross-correlation + bias: (N,Cin,H,W) -> (N,Cout,Ho,Wo)."""
    x, w = _f32(x), _f32(w)
    b = None if b is None else _f32(b)
    N, Cin, H, W = x.shape
    Cout, Cin2, K, K2 = w.shape
    if Cin2 != Cin or K2 != K:
        raise ValueError("weight shape does not match input")
    out = np.empty((N, Cout, H - K + 1, W - K + 1), dtype=np.float64)
    _check(load().oracle_conv2d(_p32(x), _p32(w), _p32(b), N, Cin, H, W, Cout, K,
                                _p64(out), _threads(nthreads)), "conv2d")
    return out


def fused_chain(x, w, b, gamma, beta, groups, eps=1e-5, nthreads=None):
    """conv -> GroupNorm -> tanh -> hardswish -> +conv -> logsumexp(dim=1).

    Returns (out (N,1,Ho,Wo), mean (N,G), rstd (N,G)), all float64.
    """
    x, w = _f32(x), _f32(w)
    b = None if b is None else _f32(b)
    gamma = None if gamma is None else _f32(gamma)
    beta = None if beta is None else _f32(beta)
    N, Cin, H, W = x.shape
    Cout, Cin2, K, K2 = w.shape
    if Cin2 != Cin or K2 != K:
        raise ValueError("weight shape does not match input")
    Ho, Wo = H - K + 1, W - K + 1
    out = np.empty((N, 1, Ho, Wo), dtype=np.float64)
    mean = np.empty((N, groups), dtype=np.float64)
    rstd = np.empty((N, groups), dtype=np.float64)
    _check(load().oracle_fused_chain(_p32(x), _p32(w), _p32(b), _p32(gamma),
                                     _p32(beta), N, Cin, H, W, Cout, K, groups,
                                     float(eps), _p64(out), _p64(mean), _p64(rstd),
                                     _threads(nthreads)), "fused_chain")
    return out, mean, rstd
