"""Builds libmm.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m dense_bf16_gemm_amd.build

Compiler resource remarks (registers, spills, scratch, LDS per kernel) are
kept in ``_build/resource_usage.txt`` next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmm.so")
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


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    with open(REMARKS, "w") as f:
        f.write(res.stderr)
    if res.returncode != 0:
        errs = [ln for ln in res.stderr.splitlines() if "error" in ln]
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs[:40]))
    os.replace(tmp, LIB)
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
