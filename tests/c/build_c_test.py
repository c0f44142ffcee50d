"""Builds tests/c/mm_from_c: the C-ABI test program (plain C11 with gcc),
linked against libmm.so, the oracle's liboracle.so and the HIP runtime.
Run by __graft_entry__.build() after both libraries are built."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "mm_from_c")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.join(ROOT, "dense_bf16_gemm_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           "-o", BIN + ".tmp", os.path.join(HERE, "mm_from_c.c"),
           "-L", pkg, "-l:libmm.so", "-L", orc, "-l:liboracle.so",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           # found next to the program wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../dense_bf16_gemm_amd:$ORIGIN/../../oracle:" + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
