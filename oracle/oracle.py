"""Python driver for the plain-C fp64 oracle in oracle.c.

TEST INFRASTRUCTURE ONLY.  The product library never imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the GPU path: it links nothing from the library and
marshals numpy arrays into liboracle.so, built from oracle.c with gcc.

Every function returns float64 results.  See oracle.c for the definitions and
the page passages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no
    contraction, so each addition rounds exactly once in binary64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        lib.oracle_w4_dequant.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_w4_gemv.argtypes = [P, I, P, P, P, I, I, I, I, P]
        lib.oracle_w4_gemv_cols.argtypes = [P, I, P, P, P, I, I, I, I, P, I, P]
        lib.oracle_w2t_dequant.argtypes = [P, P, I, I, I, P]
        lib.oracle_w2t_gemv.argtypes = [P, I, P, P, I, I, I, I, P]
        lib.oracle_w2t_gemv_cols.argtypes = [P, I, P, P, I, I, I, I, P, I, P]
        lib.oracle_w16_gemv.argtypes = [P, I, P, I, I, I, P]
        lib.oracle_w16_gemv_cols.argtypes = [P, I, P, I, I, I, P, I, P]
        lib.oracle_e2m1_to_f64.argtypes = [I]
        lib.oracle_e2m1_to_f64.restype = ctypes.c_double
        lib.oracle_e8m0_to_f64.argtypes = [I]
        lib.oracle_e8m0_to_f64.restype = ctypes.c_double
        lib.oracle_mx_dequant.argtypes = [P, P, I, I, P]
        lib.oracle_mx_gemv.argtypes = [P, I, P, P, I, I, I, P]
        lib.oracle_mx_gemv_cols.argtypes = [P, I, P, P, I, I, I, P, I, P]
        for f in ("oracle_w4_dequant", "oracle_w4_gemv", "oracle_w4_gemv_cols",
                  "oracle_w2t_dequant", "oracle_w2t_gemv", "oracle_w2t_gemv_cols",
                  "oracle_w16_gemv", "oracle_w16_gemv_cols", "oracle_mx_dequant",
                  "oracle_mx_gemv", "oracle_mx_gemv_cols"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc == -2:
        raise ValueError(f"{what}: ternary code 3 present (invalid input)")
    if rc != 0:
        raise ValueError(f"{what}: invalid shape or arguments (rc={rc})")


def num_threads() -> int:
    return _load().oracle_num_threads()


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def w4_dequant(qweight, scales, zeros, N: int, K: int, group: int) -> np.ndarray:
    """W[K][N] = (q - z) * s in float64."""
    q, s, z = _c(qweight, np.int32), _c(scales, np.uint16), _c(zeros, np.int32)
    W = np.empty((K, N), dtype=np.float64)
    _check(_load().oracle_w4_dequant(_ptr(q), _ptr(s), _ptr(z), N, K, group, _ptr(W)), "w4_dequant")
    return W


def w4_gemv(x, x_dtype: str, qweight, scales, zeros, M: int, N: int, K: int, group: int,
            cols=None) -> np.ndarray:
    """y[M][N] (or y[M][len(cols)] for the listed columns) = x . W in float64."""
    xb = _c(x, np.uint16)
    q, s, z = _c(qweight, np.int32), _c(scales, np.uint16), _c(zeros, np.int32)
    bf = 1 if x_dtype == "bf16" else 0
    lib = _load()
    if cols is None:
        y = np.empty((M, N), dtype=np.float64)
        _check(lib.oracle_w4_gemv(_ptr(xb), bf, _ptr(q), _ptr(s), _ptr(z), M, N, K, group, _ptr(y)),
               "w4_gemv")
    else:
        c = _c(cols, np.int64)
        y = np.empty((M, len(c)), dtype=np.float64)
        _check(lib.oracle_w4_gemv_cols(_ptr(xb), bf, _ptr(q), _ptr(s), _ptr(z), M, N, K, group,
                                       _ptr(c), len(c), _ptr(y)), "w4_gemv_cols")
    return y


def w2t_dequant(codes, scales, N: int, K: int, group: int) -> np.ndarray:
    """W[K][N] = (c - 1) * s in float64."""
    c, s = _c(codes, np.int32), _c(scales, np.uint16)
    W = np.empty((K, N), dtype=np.float64)
    _check(_load().oracle_w2t_dequant(_ptr(c), _ptr(s), N, K, group, _ptr(W)), "w2t_dequant")
    return W


def w2t_gemv(x, x_dtype: str, codes, scales, M: int, N: int, K: int, group: int,
             cols=None) -> np.ndarray:
    xb = _c(x, np.uint16)
    c, s = _c(codes, np.int32), _c(scales, np.uint16)
    bf = 1 if x_dtype == "bf16" else 0
    lib = _load()
    if cols is None:
        y = np.empty((M, N), dtype=np.float64)
        _check(lib.oracle_w2t_gemv(_ptr(xb), bf, _ptr(c), _ptr(s), M, N, K, group, _ptr(y)),
               "w2t_gemv")
    else:
        cc = _c(cols, np.int64)
        y = np.empty((M, len(cc)), dtype=np.float64)
        _check(lib.oracle_w2t_gemv_cols(_ptr(xb), bf, _ptr(c), _ptr(s), M, N, K, group,
                                        _ptr(cc), len(cc), _ptr(y)), "w2t_gemv_cols")
    return y


def w16_gemv(x, dtype: str, w, M: int, N: int, K: int, cols=None) -> np.ndarray:
    """y[M][N] (or the listed columns) = x . w^T in float64, for 16-bit
    weights w[N][K] of the same dtype as x (bit patterns as uint16)."""
    xb, wb = _c(x, np.uint16), _c(w, np.uint16)
    bf = 1 if dtype == "bf16" else 0
    lib = _load()
    if cols is None:
        y = np.empty((M, N), dtype=np.float64)
        _check(lib.oracle_w16_gemv(_ptr(xb), bf, _ptr(wb), M, N, K, _ptr(y)), "w16_gemv")
    else:
        c = _c(cols, np.int64)
        y = np.empty((M, len(c)), dtype=np.float64)
        _check(lib.oracle_w16_gemv_cols(_ptr(xb), bf, _ptr(wb), M, N, K, _ptr(c), len(c), _ptr(y)),
               "w16_gemv_cols")
    return y


def e2m1_to_f64(code: int) -> float:
    """Value of a 4-bit E2M1 element code (MXFP4 element)."""
    return _load().oracle_e2m1_to_f64(int(code))


def e8m0_to_f64(code: int) -> float:
    """Value of an 8-bit E8M0 scale code: 2^(code - 127), NaN for 255."""
    return _load().oracle_e8m0_to_f64(int(code))


def mx_dequant(qweight, scales, N: int, K: int) -> np.ndarray:
    """MXFP4 weights w[N][K] in float64 from qweight uint8 [N][K/2] (low
    nibble = even k) and E8M0 scales uint8 [N][K/32]."""
    q, s = _c(qweight, np.uint8), _c(scales, np.uint8)
    w = np.empty((N, K), dtype=np.float64)
    _check(_load().oracle_mx_dequant(_ptr(q), _ptr(s), N, K, _ptr(w)), "mx_dequant")
    return w


def mx_gemv(x, x_dtype: str, qweight, scales, M: int, N: int, K: int, cols=None) -> np.ndarray:
    """y[M][N] (or the listed columns) = x . w^T in float64 for MXFP4 w."""
    xb, q, s = _c(x, np.uint16), _c(qweight, np.uint8), _c(scales, np.uint8)
    bf = 1 if x_dtype == "bf16" else 0
    lib = _load()
    if cols is None:
        y = np.empty((M, N), dtype=np.float64)
        _check(lib.oracle_mx_gemv(_ptr(xb), bf, _ptr(q), _ptr(s), M, N, K, _ptr(y)), "mx_gemv")
    else:
        c = _c(cols, np.int64)
        y = np.empty((M, len(c)), dtype=np.float64)
        _check(lib.oracle_mx_gemv_cols(_ptr(xb), bf, _ptr(q), _ptr(s), M, N, K, _ptr(c), len(c),
                                       _ptr(y)), "mx_gemv_cols")
    return y
