"""Builds libmm.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m dense_bf16_gemm_amd.build

Compiler resource remarks (registers, spills, scratch, LDS per kernel) are
kept in ``_build/resource_usage.txt`` next to this file.

A second library, ``libmm_fullsync.so``, is built from the same sources with
MM_DEBUG_FULL_SYNC: the slab kernel then drains every copy and waits at a
barrier before each super-step.  It is a race check for the tests (its
results must equal libmm.so's bit for bit), never the product.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmm.so")
LIB_FULLSYNC = os.path.join(HERE, "libmm_fullsync.so")
BUILD_DIR = os.path.join(HERE, "_build")
REMARKS = os.path.join(BUILD_DIR, "resource_usage.txt")
SOURCES = ["mm_api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Rpass-analysis=kernel-resource-usage",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _command(out: str, defines=()) -> list:
    return [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
            "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    """Builds libmm.so and the race-check libmm_fullsync.so (two hipcc runs
    side by side); returns the path of libmm.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for lib, defines in ((LIB, ()), (LIB_FULLSYNC, ("MM_DEBUG_FULL_SYNC",))):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = _command(tmp, defines)
        if verbose:
            print(" ".join(cmd), flush=True)
        # compiler output to a file (a pipe could fill while the other job runs)
        log = REMARKS if lib == LIB else os.path.join(BUILD_DIR, "fullsync_build.txt")
        with open(log, "w") as f:
            proc = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=f)
        jobs.append((lib, tmp, log, proc))
    failed = []
    for lib, tmp, log, proc in jobs:
        proc.wait()
        with open(log) as f:
            err = f.read()
        if proc.returncode != 0:
            errs = [ln for ln in err.splitlines() if "error" in ln]
            failed.append(f"hipcc failed for {os.path.basename(lib)}:\n" + "\n".join(errs[:40]))
        else:
            os.replace(tmp, lib)
    if failed:
        raise RuntimeError("\n".join(failed))
    return LIB


def resource_usage(path: str = REMARKS):
    """Parses the resource remarks into {kernel: {field: int}} (True / False
    fields, such as "Dynamic Stack", as 1 / 0)."""
    out = {}
    cur = None
    with open(path) as f:
        for line in f:
            if "remark:" not in line:
                continue
            body = line.split("remark:", 1)[1].strip()
            body = body.replace("[-Rpass-analysis=kernel-resource-usage]", "").strip()
            if body.startswith("Function Name:"):
                cur = body.split(":", 1)[1].strip()
                out[cur] = {}
            elif cur is not None and ":" in body:
                key, val = body.rsplit(":", 1)
                val = {"True": "1", "False": "0"}.get(val.strip(), val.strip())
                try:
                    out[cur][key.strip()] = int(val)
                except ValueError:
                    pass
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
