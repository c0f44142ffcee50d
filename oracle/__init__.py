"""CPU oracle for the bf16 GEMM hot path -- test infrastructure only.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The product path (``dense_bf16_gemm_amd``) never
does, and this module never imports the product package: the two share no
code.  Inputs are plain numpy arrays of bf16 bit patterns (``uint16``).

The arithmetic lives in ``oracle.c`` (plain C + OpenMP, built with gcc); see
the header there for what is computed and which passages of the pages each
part follows.  This file only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

LAYOUTS = {"nn": 0, "nt": 1, "tn": 2, "tt": 3}
EPILOGUES = {
    "none": 0,
    "bias": 1,
    "gelu_tanh": 2,
    "bias_gelu_tanh": 3,
    "swiglu": 4,
    "glu_identity": 5,
}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no HIP, no -ffast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-std=c11", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f32p = ctypes.POINTER(ctypes.c_float)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_gemm.argtypes = [u16p, u16p, u16p, u16p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                i64, i64, f32p, u16p, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_points.argtypes = [u16p, u16p, u16p, u16p, i64, i64, i64, ctypes.c_int,
                                       ctypes.c_int, i64p, i64p, i64, f32p, u16p, ctypes.c_int]
    lib.oracle_gemm_points.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [f32p, u16p, i64]
    lib.oracle_gelu_tanh.argtypes = [f32p, f32p, i64]
    lib.oracle_silu_mul.argtypes = [f32p, f32p, f32p, i64]
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle operands are uint16 arrays of bf16 bit patterns")
    return a


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _shapes(A, B, layout):
    lay = LAYOUTS[layout]
    if lay in (2, 3):
        K, M = A.shape
    else:
        M, K = A.shape
    if lay in (1, 3):
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError(f"K mismatch: A gives {K}, B gives {Kb}")
    return lay, M, N, K


def gemm(A, B, layout="nn", epilogue="none", bias=None, B2=None, rows=None, nthreads=0,
         timed=False):
    """Rows ``rows=(begin, end)`` (default: all) of epi(op(A).op(B) [+bias]).

    Returns ``(y, bits)``: the fp32 result and its RNE bf16 bit patterns; with
    ``timed=True`` also the seconds spent in the contraction+epilogue loops.
    """
    lib = _load()
    A, B, B2, bias = _u16(A), _u16(B), _u16(B2), _u16(bias)
    lay, M, N, K = _shapes(A, B, layout)
    if B2 is not None and B2.shape != B.shape:
        raise ValueError("B2 must have B's shape")
    if bias is not None and bias.shape != (N,):
        raise ValueError("bias must have shape (N,)")
    rb, re = (0, M) if rows is None else rows
    y = np.empty((re - rb, N), np.float32)
    bits = np.empty((re - rb, N), np.uint16)
    secs = ctypes.c_double(0.0)
    rc = lib.oracle_gemm(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                         _ptr(B2, ctypes.c_uint16), _ptr(bias, ctypes.c_uint16), M, N, K, lay,
                         EPILOGUES[epilogue], rb, re, _ptr(y, ctypes.c_float),
                         _ptr(bits, ctypes.c_uint16), int(nthreads), ctypes.byref(secs))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed with code {rc}")
    if timed:
        return y, bits, secs.value
    return y, bits


def points(A, B, rows, cols, layout="nn", epilogue="none", bias=None, B2=None, nthreads=0):
    """Outputs at (rows[p], cols[p]) by the literal per-element k loop."""
    lib = _load()
    A, B, B2, bias = _u16(A), _u16(B), _u16(B2), _u16(bias)
    lay, M, N, K = _shapes(A, B, layout)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    n = rows.shape[0]
    y = np.empty(n, np.float32)
    bits = np.empty(n, np.uint16)
    rc = lib.oracle_gemm_points(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                _ptr(B2, ctypes.c_uint16), _ptr(bias, ctypes.c_uint16), M, N, K,
                                lay, EPILOGUES[epilogue], _ptr(rows, ctypes.c_int64),
                                _ptr(cols, ctypes.c_int64), n, _ptr(y, ctypes.c_float),
                                _ptr(bits, ctypes.c_uint16), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_points failed with code {rc}")
    return y, bits


def round_bf16(x):
    """RNE fp32 -> bf16 bit patterns, as the oracle rounds its outputs."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.oracle_round_bf16(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def gelu_tanh(t):
    lib = _load()
    t = np.ascontiguousarray(t, dtype=np.float32)
    y = np.empty(t.shape, np.float32)
    lib.oracle_gelu_tanh(_ptr(t, ctypes.c_float), _ptr(y, ctypes.c_float), t.size)
    return y


def silu_mul(g, u):
    lib = _load()
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    y = np.empty(g.shape, np.float32)
    lib.oracle_silu_mul(_ptr(g, ctypes.c_float), _ptr(u, ctypes.c_float), _ptr(y, ctypes.c_float),
                        g.size)
    return y


def max_threads() -> int:
    return int(_load().oracle_max_threads())
