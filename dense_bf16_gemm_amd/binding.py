"""ctypes binding of libmm.so (declared in include/mm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback path: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmm.so")
FULLSYNC_LIB_PATH = os.path.join(HERE, "libmm_fullsync.so")

MM_OK, MM_ERR_INVALID_VALUE, MM_ERR_UNSUPPORTED, MM_ERR_MISALIGNED, MM_ERR_HIP = range(5)
LAYOUTS = {"nn": 0, "nt": 1, "tn": 2, "tt": 3}
EPILOGUES = {"none": 0, "bias": 1, "gelu_tanh": 2, "bias_gelu_tanh": 3}
OUT_DTYPES = {"bf16": 0, "f32": 1}
GLU_ACTS = {"silu": 0, "identity": 1}

EXPORTS = (
    "mm_matmul", "mm_linear", "mm_ffn_swiglu", "mm_ffn_glu", "mm_set_config",
    "mm_describe_config", "mm_debug_schedule", "mm_status_string", "mm_last_error",
    "mm_workspace_size", "mm_matmul_ws", "mm_linear_ws", "mm_matmul_batched", "mm_linear_batched",
    "mm_linear_preact", "mm_matmul_noalloc",
)

_lib = None


class MMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load(path: str = LIB_PATH):
    """Loads libmm.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = open_library(path)
    return _lib


def open_library(path: str):
    """Opens one build of the library (libmm.so, or the race-check build
    libmm_fullsync.so next to it) with its prototypes set; raises if it is
    missing.  Each build is opened with its own symbol scope."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m dense_bf16_gemm_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mm_matmul.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.mm_linear.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.mm_ffn_swiglu.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.mm_ffn_glu.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp]
    lib.mm_workspace_size.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(ctypes.c_int64)]
    lib.mm_matmul_ws.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp, i64, vp]
    lib.mm_matmul_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.mm_linear_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, vp, i64, vp]
    lib.mm_matmul_batched.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    lib.mm_linear_batched.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    lib.mm_linear_preact.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.mm_set_config.argtypes = [ctypes.c_char_p]
    lib.mm_describe_config.argtypes = [ci, i64, i64, i64, ci, ctypes.c_char_p, i64]
    lib.mm_debug_schedule.argtypes = [ci, i64, i64, i64, ci, i64, ctypes.POINTER(ctypes.c_int32), i64,
                                      ctypes.POINTER(ctypes.c_int64)]
    for name in ("mm_matmul", "mm_linear", "mm_ffn_swiglu", "mm_ffn_glu", "mm_set_config",
                 "mm_describe_config", "mm_debug_schedule", "mm_workspace_size", "mm_matmul_ws",
                 "mm_linear_ws", "mm_matmul_batched", "mm_linear_batched", "mm_linear_preact",
                 "mm_matmul_noalloc"):
        getattr(lib, name).restype = ci
    lib.mm_status_string.argtypes = [ci]
    lib.mm_status_string.restype = ctypes.c_char_p
    lib.mm_last_error.argtypes = []
    lib.mm_last_error.restype = ctypes.c_char_p
    return lib


def check(status: int, what: str) -> None:
    if status != MM_OK:
        lib = load()
        raise MMError(status, f"{what}: {lib.mm_status_string(status).decode()}: "
                              f"{lib.mm_last_error().decode()}")


def set_config(spec: Optional[str]) -> None:
    """Replaces the tile-configuration heuristic (None/"" restores it)."""
    check(load().mm_set_config(spec.encode() if spec else None), "mm_set_config")


def workspace_size(form: str, M: int, N: int, K: int, layout: str = "nt") -> int:
    """Bytes of split-K workspace a call of this shape may use on the current
    device (0: none)."""
    n = ctypes.c_int64(0)
    check(load().mm_workspace_size(1 if form == "ffn" else 0, M, N, K, LAYOUTS[layout],
                                   ctypes.byref(n)), "mm_workspace_size")
    return n.value


def describe_config(form: str, M: int, N: int, K: int, layout: str = "nt") -> str:
    buf = ctypes.create_string_buffer(256)
    check(load().mm_describe_config(1 if form == "ffn" else 0, M, N, K, LAYOUTS[layout], buf, 256),
          "mm_describe_config")
    return buf.value.decode()


def debug_schedule(form: str, M: int, N: int, K: int, grid: int, layout: str = "nt"):
    """The persistent tile order as a list of (block, local_i, tile_m, tile_n, k_desc)."""
    lib = load()
    count = ctypes.c_int64(0)
    f = 1 if form == "ffn" else 0
    check(lib.mm_debug_schedule(f, M, N, K, LAYOUTS[layout], grid, None, 0, ctypes.byref(count)),
          "mm_debug_schedule")
    n = count.value
    buf = (ctypes.c_int32 * (5 * max(n, 1)))()
    check(lib.mm_debug_schedule(f, M, N, K, LAYOUTS[layout], grid, buf, n, ctypes.byref(count)),
          "mm_debug_schedule")
    return [tuple(buf[5 * i:5 * i + 5]) for i in range(n)]
