"""MI355X-native bf16 GEMM: MatmulOp / LinearOp forms with fused epilogues.

The operations run in hand-written HIP kernels for gfx950 behind the C ABI in
``include/mm.h`` (``libmm.so``); this package only marshals arguments to it.
The library is loaded on first use and its absence is an error.
"""
from .gemm import (bmm, ffn_glu, ffn_swiglu, linear, linear_batched, linear_preact, matmul,  # noqa: F401
                   release_workspaces)
from .binding import describe_config, set_config  # noqa: F401
