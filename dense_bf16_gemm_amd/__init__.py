"""MI355X-native bf16 GEMM: MatmulOp / LinearOp forms with fused epilogues.

The operations run in hand-written HIP kernels for gfx950 behind the C ABI in
``include/mm.h`` (``libmm.so``); this package only marshals arguments to it.
"""
