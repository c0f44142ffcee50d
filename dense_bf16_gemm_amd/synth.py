"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and describes workload shapes; it holds
none of the GEMM's arithmetic and imports neither the HIP library nor the
oracle.  Every tensor is generated on the CPU from a fixed seed (except the
> 2^31-element stress operand, drawn on the device from a seeded generator),
so the GPU path and the oracle see the same bf16 bit patterns.

Value distributions follow the pages' test inputs (PR "Implement persistent
matmul scheduling", reviewer guide: operands drawn with randn in bf16), scaled
per workload so that outputs stay O(1): sigma is a standard deviation, and a
weight of "variance 1/K" gets sigma = K**-0.5.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import torch


def randn_bf16(shape, sigma: float, seed: int) -> torch.Tensor:
    """N(0, sigma^2) drawn in fp32 from ``seed`` on the CPU, then rounded to bf16."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(float(sigma))
    return x.to(torch.bfloat16)


def randint_bf16(shape, lo: int, hi: int, seed: int) -> torch.Tensor:
    """Uniform integers in [lo, hi] (inclusive) as bf16 (exact for |v| <= 256)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, dtype=torch.int32).to(torch.bfloat16)


def sparse_pm1_rows(rows: int, k: int, nnz: int, seed: int) -> torch.Tensor:
    """[rows, k] bf16 with ``min(nnz, k)`` entries of +-1 per row at random columns."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    nnz = min(nnz, k)
    out = torch.zeros(rows, k, dtype=torch.float32)
    if rows == 0 or k == 0 or nnz == 0:
        return out.to(torch.bfloat16)
    cols = torch.argsort(torch.rand(rows, k, generator=g), dim=1)[:, :nnz]
    signs = torch.randint(0, 2, (rows, nnz), generator=g).to(torch.float32).mul_(2).sub_(1)
    out.scatter_(1, cols, signs)
    return out.to(torch.bfloat16)


def bits(t: torch.Tensor):
    """The bf16 bit patterns of a CPU tensor as a numpy uint16 array (no copy)."""
    import numpy as np

    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    sigma: float
    seed: int


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity workload: the op form, sizes, layout and inputs."""

    name: str
    form: str  # "matmul" | "linear" | "ffn"
    M: int
    N: int
    K: int
    layout: str  # op(A).op(B) letters, see include/mm.h
    epilogue: str  # "none" | "bias" | "gelu_tanh" | "bias_gelu_tanh" | "swiglu"
    out_dtype: str  # "bf16" | "f32"
    tensors: Tuple[TensorSpec, ...]

    @property
    def flops(self) -> int:
        """Algorithmic flops: 2*M*N*K per GEMM (two GEMMs for the FFN)."""
        g = 2 if self.form == "ffn" else 1
        return 2 * self.M * self.N * self.K * g

    @property
    def algorithmic_bytes(self) -> int:
        """Each operand read once plus the output written once."""
        total = 0
        for t in self.tensors:
            n = 1
            for s in t.shape:
                n *= s
            total += 2 * n
        return total + self.M * self.N * (4 if self.out_dtype == "f32" else 2)

    def make(self) -> Dict[str, torch.Tensor]:
        return {t.name: randn_bf16(t.shape, t.sigma, t.seed) for t in self.tensors}


# The five workloads: a small plain matmul, linear+bias+GELU at two scales, the
# Llama-FFN horizontal fusion, and a long-K non-tile-divisible matmul whose B is
# a transposed view.  Then the plain matmul at 8192^3 in each operand storage
# (A as given or stored [K][M] as "At", B as given or stored [N][K] as "Bt"),
# for the layout comparison.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("matmul_nn_256", "matmul", 256, 256, 256, "nn", "none", "bf16",
                 (TensorSpec("A", (256, 256), 1.0, 101), TensorSpec("B", (256, 256), 1.0, 102))),
        Workload("linear_bias_gelu_4096", "linear", 4096, 4096, 4096, "nt", "bias_gelu_tanh", "bf16",
                 (TensorSpec("x", (4096, 4096), 1.0, 201), TensorSpec("W", (4096, 4096), 2.0 ** -6, 202),
                  TensorSpec("bias", (4096,), 1.0, 203))),
        Workload("linear_bias_gelu_8192", "linear", 8192, 8192, 8192, "nt", "bias_gelu_tanh", "bf16",
                 (TensorSpec("x", (8192, 8192), 1.0, 301), TensorSpec("W", (8192, 8192), 8192 ** -0.5, 302),
                  TensorSpec("bias", (8192,), 1.0, 303))),
        Workload("ffn_swiglu_8192x14336x4096", "ffn", 8192, 14336, 4096, "nt", "swiglu", "bf16",
                 (TensorSpec("x", (8192, 4096), 1.0, 401), TensorSpec("W_gate", (14336, 4096), 2.0 ** -6, 402),
                  TensorSpec("W_up", (14336, 4096), 2.0 ** -6, 403))),
        Workload("matmul_longk_nt_f32_2047x3001x65536", "matmul", 2047, 3001, 65536, "nt", "none", "f32",
                 (TensorSpec("A", (2047, 65536), 1.0, 501), TensorSpec("Bt", (3001, 65536), 2.0 ** -8, 502))),
    ] + [
        Workload(f"matmul_{lay}_8192", "matmul", 8192, 8192, 8192, lay, "none", "bf16",
                 (TensorSpec("At" if lay[0] == "t" else "A", (8192, 8192), 1.0, 601 + 2 * i),
                  TensorSpec("Bt" if lay[1] == "t" else "B", (8192, 8192), 8192 ** -0.5, 602 + 2 * i)))
        for i, lay in enumerate(("nn", "nt", "tn", "tt"))
    ]
}

# Shapes measured for one design question each (bench.py --workload), not
# parity workloads: an 8192 x 8192 output (four tiles per workgroup) with
# K = 65536, whose 32 MiB K panels are far larger than an XCD's 4 MiB L2 --
# where the direction of each tile's K loop could matter; and a decode-step
# product (16 activation rows against a 448 MiB weight, larger than the
# 256 MiB last-level cache), bound by reading the weight once.
EXTRA_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("matmul_nt_8192x8192x65536", "matmul", 8192, 8192, 65536, "nt", "none", "bf16",
                 (TensorSpec("A", (8192, 65536), 1.0, 701), TensorSpec("Bt", (8192, 65536), 2.0 ** -8, 702))),
        Workload("linear_bias_decode_16x28672x8192", "linear", 16, 28672, 8192, "nt", "bias", "bf16",
                 (TensorSpec("x", (16, 8192), 1.0, 801), TensorSpec("W", (28672, 8192), 8192 ** -0.5, 802),
                  TensorSpec("bias", (28672,), 1.0, 803))),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "linear_bias_gelu_8192"


def mapping_operands(M: int, N: int, K: int, layout: str, seed: int, gated: bool = False,
                     with_bias: bool = False) -> Dict[str, Optional[torch.Tensor]]:
    """Integer-valued operands whose fp32 sums are exact in any order.

    A has 32 entries of +-1 per output row, B (and B2) are integers in
    [-4, 4], bias integers in [-64, 64]: every output is an integer of
    magnitude <= 192, exact in fp32 and in bf16, so a misplaced row, column or
    K slice changes the result bits.  Returned in storage layout.
    """
    a = sparse_pm1_rows(M, K, 32, seed)  # op(A) as [M, K]
    b = randint_bf16((K, N), -4, 4, seed + 1)  # op(B) as [K, N]
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["A"] = a.t().contiguous() if layout in ("tn", "tt") else a
    out["B"] = b.t().contiguous() if layout in ("nt", "tt") else b
    out["B2"] = None
    if gated:
        b2 = randint_bf16((K, N), -4, 4, seed + 2)
        out["B2"] = b2.t().contiguous() if layout in ("nt", "tt") else b2
    out["bias"] = randint_bf16((N,), -64, 64, seed + 3) if with_bias else None
    return out


def dense_int_operands(M: int, N: int, K: int, layout: str, seed: int, lo: int = -2, hi: int = 2):
    """Dense integer operands for fp32-output mapping tests (|out| <= 4K < 2^24)."""
    a = randint_bf16((M, K), lo, hi, seed)
    b = randint_bf16((K, N), lo, hi, seed + 1)
    A = a.t().contiguous() if layout in ("tn", "tt") else a
    B = b.t().contiguous() if layout in ("nt", "tt") else b
    return A, B


def sample_points(M: int, N: int, n: int, seed: int, tile: Tuple[int, int] = (256, 256)) -> Tuple[List[int], List[int]]:
    """``n`` random output coordinates plus the four corners of every edge tile row/col."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    rows = torch.randint(0, M, (n,), generator=g).tolist()
    cols = torch.randint(0, N, (n,), generator=g).tolist()
    # the last row/column (ragged edges) and tile-boundary neighbours
    extra_r = sorted({0, M - 1} | {min(M - 1, r) for r in range(tile[0] - 1, M + 1, tile[0])}
                     | {min(M - 1, r + 1) for r in range(tile[0] - 1, M, tile[0])})
    extra_c = sorted({0, N - 1} | {min(N - 1, c) for c in range(tile[1] - 1, N + 1, tile[1])}
                     | {min(N - 1, c + 1) for c in range(tile[1] - 1, N, tile[1])})
    for r in extra_r:
        rows.append(r)
        cols.append(int(torch.randint(0, N, (1,), generator=g)))
    for c in extra_c:
        cols.append(c)
        rows.append(int(torch.randint(0, M, (1,), generator=g)))
    return rows, cols
