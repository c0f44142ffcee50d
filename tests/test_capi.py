"""Host-side checks of libmm.so: it loads without a GPU, exports every
function include/mm.h declares, rejects bad arguments before touching HIP,
and its tile order covers every output tile exactly once.

No test here launches a kernel, and no call here passes validation with a
pointer that is not real device memory.
"""
import os
import re

import pytest

from dense_bf16_gemm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mm.h")

# fake, never dereferenced, 256-byte aligned addresses
PA, PB, PB2, PBIAS, POUT = (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000)


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mm_status|const char\*)\s+(mm_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_race_check_build_loads_and_exports_every_declared_symbol():
    """The MM_DEBUG_FULL_SYNC build (used only by the GPU race check) is
    built beside libmm.so and has the same interface."""
    other = binding.open_library(binding.FULLSYNC_LIB_PATH)
    for name in declared_functions():
        assert hasattr(other, name), name
    assert other.mm_status_string(0).decode() == "MM_OK"


def test_status_strings(lib):
    for code, name in enumerate(["MM_OK", "MM_ERR_INVALID_VALUE", "MM_ERR_UNSUPPORTED",
                                 "MM_ERR_MISALIGNED", "MM_ERR_HIP"]):
        assert lib.mm_status_string(code).decode() == name
    assert lib.mm_status_string(99).decode() == "MM_ERR_UNKNOWN"


def mm(lib, A=PA, B=PB, out=POUT, M=64, N=64, K=64, layout=1, out_dtype=0):
    return lib.mm_matmul(A, B, out, M, N, K, layout, out_dtype, None)


def lin(lib, x=PA, W=PB, bias=PBIAS, out=POUT, M=64, N=64, K=64, layout=1, epi=3):
    return lib.mm_linear(x, W, bias, out, M, N, K, layout, epi, None)


def test_argument_errors_return_before_any_device_call(lib):
    E = binding
    assert mm(lib, A=None) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, B=None) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, out=None) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, M=-1) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, K=-5) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, layout=7) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, out_dtype=3) == E.MM_ERR_INVALID_VALUE
    # K == 0 is the empty sum: its operands may be null, never its output
    assert mm(lib, K=0, A=None, B=None, out=None) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, K=0, A=None, B=None) not in (E.MM_ERR_INVALID_VALUE, E.MM_ERR_UNSUPPORTED,
                                                 E.MM_ERR_MISALIGNED)
    assert lin(lib, K=0, x=None, W=None, bias=None, epi=1) == E.MM_ERR_INVALID_VALUE  # bias still needed
    assert mm(lib, M=1 << 31) == E.MM_ERR_UNSUPPORTED
    # alignment of operand pointers and of contiguous extents
    assert mm(lib, A=PA + 2) == E.MM_ERR_MISALIGNED
    assert mm(lib, B=PB + 8) == E.MM_ERR_MISALIGNED
    assert mm(lib, K=60) == E.MM_ERR_MISALIGNED  # NT: K is contiguous for both
    assert mm(lib, N=60, layout=0) == E.MM_ERR_MISALIGNED  # NN: B's rows are N long
    assert mm(lib, M=60, layout=2) == E.MM_ERR_MISALIGNED  # TN: A's rows are M long
    assert mm(lib, out=POUT + 2, out_dtype=1) == E.MM_ERR_MISALIGNED
    # output overlapping an input
    assert mm(lib, out=PA + 64) == E.MM_ERR_INVALID_VALUE
    assert mm(lib, out=PB - 64) == E.MM_ERR_INVALID_VALUE
    # linear: epilogue enum and bias requirement
    assert lin(lib, epi=9) == E.MM_ERR_INVALID_VALUE
    assert lin(lib, bias=None, epi=1) == E.MM_ERR_INVALID_VALUE
    assert lin(lib, bias=None, epi=3) == E.MM_ERR_INVALID_VALUE
    assert lin(lib, bias=PBIAS + 1) == E.MM_ERR_MISALIGNED
    assert lin(lib, out=PBIAS) == E.MM_ERR_INVALID_VALUE
    # FFN
    assert lib.mm_ffn_swiglu(PA, PB, None, POUT, 64, 64, 64, None) == E.MM_ERR_INVALID_VALUE
    assert lib.mm_ffn_glu(PA, PB, PB2, POUT, 64, 64, 64, 5, None) == E.MM_ERR_INVALID_VALUE
    assert lib.mm_ffn_swiglu(PA, PB, PB2, POUT, 64, 64, 36, None) == E.MM_ERR_MISALIGNED


def test_empty_output_is_a_no_op(lib):
    # M == 0 or N == 0 succeeds without a device or a launch
    assert mm(lib, M=0) == binding.MM_OK
    assert mm(lib, N=0, A=None, B=None, out=None) == binding.MM_OK
    assert lin(lib, M=0, bias=None) == binding.MM_OK
    assert lib.mm_ffn_swiglu(None, None, None, None, 0, 64, 64, None) == binding.MM_OK


def test_config_override_and_rejection(lib):
    try:
        binding.set_config("BM=128,BN=128,WM=2,WN=2,G=4,XCD=0,KALT=0")
        assert binding.describe_config("linear", 8192, 8192, 8192).startswith(
            "BM=128,BN=128,WM=2,WN=2,G=4,XCD=0,KALT=0")
        for bad in ("BM=100", "BM=256,BN=256,WM=3,WN=2", "FOO=1", "BM=", "G=0", "KALT=7"):
            with pytest.raises(binding.MMError) as e:
                binding.set_config(bad)
            assert e.value.status == binding.MM_ERR_UNSUPPORTED
        # a rejected string leaves the previous override in place
        assert binding.describe_config("linear", 8192, 8192, 8192).startswith("BM=128,BN=128")
    finally:
        binding.set_config(None)
    assert binding.describe_config("linear", 8192, 8192, 8192).startswith("BM=256,BN=256")


def test_heuristic_choices():
    assert binding.describe_config("linear", 8192, 8192, 8192).startswith("BM=256,BN=256")
    # 256 x 256 tiles run the whole-line slab kernel when K spans two
    # super-steps of 64 (a partial last one through its ragged instances);
    # [K][N] weights and [K][M]
    # activations (NN, TN, TT) through its transpose-read forms.  Below two
    # super-steps: the 32-k pipeline for K-contiguous operands, the basic
    # kernel for the others
    assert binding.describe_config("linear", 8192, 8192, 8192).endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("ffn", 8192, 14336, 4096).endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("linear", 8192, 8192, 64).endswith("KERNEL=gemm_nt_pipe")
    assert binding.describe_config("linear", 8192, 8192, 8200).endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("linear", 8192, 8192, 136).endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("linear", 8192, 8192, 120).endswith("KERNEL=gemm_nt_pipe")
    assert binding.describe_config("ffn", 8192, 14336, 4104).endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("matmul", 8192, 8192, 8192, "nn").endswith("KERNEL=gemm_nt_slab")
    for lay in ("nn", "tn", "tt"):
        assert binding.describe_config("matmul", 8192, 8192, 8200, lay).endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("matmul", 8192, 8192, 120, "nn").endswith("KERNEL=gemm_persistent")
    assert binding.describe_config("matmul", 8192, 8192, 8192, "tn").endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("matmul", 8192, 8192, 8192, "tt").endswith("KERNEL=gemm_nt_slab")
    assert binding.describe_config("ffn", 8192, 14336, 4096).startswith("BM=256,BN=256")
    small = binding.describe_config("matmul", 256, 256, 256, "nn")
    assert small.startswith("BM=64,BN=64") and small.endswith("KERNEL=gemm_small")
    # all of K in LDS only up to K = 256; the basic kernel past it or under PIPE=0
    assert binding.describe_config("matmul", 256, 256, 264, "nn").endswith("KERNEL=gemm_persistent")
    binding.set_config("BM=64,BN=64,WM=2,WN=2,PIPE=0")
    try:
        assert binding.describe_config("matmul", 256, 256, 256, "nn").endswith("KERNEL=gemm_persistent")
    finally:
        binding.set_config(None)
    # long K turns on K-direction alternation
    assert "KALT=1" in binding.describe_config("matmul", 2047, 3001, 65536)
    assert "KALT=0" in binding.describe_config("matmul", 256, 256, 256)


def test_skinny_choices():
    """At most 32 rows against at least 8 MiB of weights take the skinny
    kernel (64 weight rows per workgroup); the slice count is the modelled
    best: none where 64-row groups already fill the CUs more than once,
    slices where they leave CUs idle."""
    assert binding.describe_config("linear", 16, 8192, 8192).endswith("SPLIT=2x64,KERNEL=gemm_skinny")
    assert binding.describe_config("linear", 16, 14336, 4096).endswith("PIPE=3,KERNEL=gemm_skinny")
    assert binding.describe_config("linear", 16, 4096, 14336).endswith("SPLIT=4x64,KERNEL=gemm_skinny")
    assert binding.describe_config("linear", 1, 4096, 1024).endswith("KERNEL=gemm_skinny")
    assert binding.describe_config("linear", 17, 8192, 8192).endswith("KERNEL=gemm_skinny")
    assert binding.describe_config("linear", 32, 14336, 4096).endswith("KERNEL=gemm_skinny")
    # 33 rows, stored-[K][N] weights, an FFN pair, too little weight, K past
    # 2^23: the tile kernels
    assert not binding.describe_config("linear", 33, 8192, 8192).endswith("gemm_skinny")
    assert not binding.describe_config("matmul", 16, 8192, 8192, "nn").endswith("gemm_skinny")
    assert not binding.describe_config("ffn", 16, 8192, 8192).endswith("gemm_skinny")
    assert not binding.describe_config("linear", 16, 1024, 2048).endswith("gemm_skinny")
    assert not binding.describe_config("linear", 1, 8, (1 << 23) + 8).endswith("gemm_skinny")
    assert binding.workspace_size("linear", 16, 14336, 4096) == 0
    assert binding.workspace_size("linear", 16, 8192, 8192) == 2 * 16 * 8192 * 4


@pytest.mark.parametrize("form,M,N,K,grid", [
    ("linear", 8192, 8192, 8192, 256),
    ("linear", 4096, 4096, 4096, 256),
    ("matmul", 2047, 3001, 65536, 256),
    ("matmul", 2047, 3001, 65536, 250),  # grid not a multiple of the XCD count
    ("ffn", 8192, 14336, 4096, 256),
    ("matmul", 1000, 3000, 64, 7),
    ("matmul", 256, 256, 256, 256),
])
def test_schedule_visits_every_tile_once(form, M, N, K, grid):
    cfg = dict(kv.split("=") for kv in binding.describe_config(form, M, N, K).split(","))
    bm, bn = int(cfg["BM"]), int(cfg["BN"])
    out_bn = bn // 2 if form == "ffn" else bn
    tiles_m, tiles_n = -(-M // bm), -(-N // out_bn)
    sched = binding.debug_schedule(form, M, N, K, grid)
    seen = [(tm, tn) for (_, _, tm, tn, _) in sched]
    assert len(seen) == tiles_m * tiles_n
    assert set(seen) == {(i, j) for i in range(tiles_m) for j in range(tiles_n)}
    G = min(grid, tiles_m * tiles_n)
    assert {b for (b, *_rest) in sched} == set(range(G))
    # each workgroup alternates K direction iff alternation is on
    kalt = cfg["KALT"] == "1"
    for (b, i, _, _, kd) in sched:
        assert kd == (1 if (kalt and i % 2 == 1) else 0)


def test_schedule_xcd_locality():
    """Workgroups the hardware places on one XCD (ids congruent mod 8) get
    consecutive tiles of one band, so they share operand panels in that
    XCD's L2."""
    sched = binding.debug_schedule("linear", 8192, 8192, 8192, 256)
    first = {b: (tm, tn) for (b, i, tm, tn, _) in sched if i == 0}
    for x in range(8):
        tiles = [first[b] for b in range(x, 256, 8)]
        rows = {tm for tm, _ in tiles}
        cols = {tn for _, tn in tiles}
        # 32 workgroups of an XCD cover a 4-row x 8-column block of tiles (band
        # height 4)
        assert len(rows) == 4 and len(cols) == 8, (x, rows, cols)


def test_batched_argument_checks():
    """Checked before any HIP call: batch < 1, negative or misaligned strides,
    overlapping output entries."""
    lib = binding.load()
    A, B, out = 4096, 8192, 1 << 30  # fake, 16-byte aligned, disjoint device addresses
    M, N, K = 64, 64, 64
    cases = [
        (0, 0, 0, M * N, binding.MM_ERR_INVALID_VALUE),          # batch 0
        (2, -8, 0, M * N, binding.MM_ERR_INVALID_VALUE),         # negative stride
        (2, 12, 0, M * N, binding.MM_ERR_MISALIGNED),            # stride not a multiple of 8
        (2, M * K, K * N, M * N - 1, binding.MM_ERR_INVALID_VALUE),  # output entries overlap
        (2, 1 << 60, 0, M * N, binding.MM_ERR_UNSUPPORTED),      # A spans 2^60 elements
        (3, 0, 0, 1 << 59, binding.MM_ERR_UNSUPPORTED),          # so does the output
    ]
    for batch, sa, sb, so, want in cases:
        st = lib.mm_matmul_batched(A, B, out, batch, M, N, K, sa, sb, so, binding.LAYOUTS["nt"], 0, None)
        assert st == want, (batch, sa, sb, so, st)


def test_preact_argument_checks():
    """mm_linear_preact rejects, before any HIP call: a non-GELU epilogue, a
    null or overlapping pre-activation output."""
    lib = binding.load()
    x, W, bias, out, pre = 4096, 8192, 1 << 20, 1 << 30, 1 << 31  # fake disjoint addresses
    M, N, K = 64, 64, 64
    nt = binding.LAYOUTS["nt"]
    E = binding.EPILOGUES
    cases = [
        (pre, E["bias"], binding.MM_ERR_INVALID_VALUE),           # no activation to precede
        (pre, E["none"], binding.MM_ERR_INVALID_VALUE),
        (None, E["bias_gelu_tanh"], binding.MM_ERR_INVALID_VALUE),  # null preact
        (out + 64, E["bias_gelu_tanh"], binding.MM_ERR_INVALID_VALUE),  # overlaps out
        (x + 2, E["gelu_tanh"], binding.MM_ERR_INVALID_VALUE),   # overlaps x
        (pre + 1, E["bias_gelu_tanh"], binding.MM_ERR_MISALIGNED),  # not element aligned
    ]
    for p, epi, want in cases:
        st = lib.mm_linear_preact(x, W, bias, out, p, M, N, K, nt, epi, None)
        assert st == want, (p, epi, st)
    # an empty product is a successful no-op
    assert lib.mm_linear_preact(x, W, bias, out, pre, 0, N, K, nt, E["bias_gelu_tanh"], None) == 0


def test_forced_band_height_is_clamped():
    """A forced band height far above the tile rows (G = 2^20 with 4096 tile
    columns: G * tiles_n would pass 2^32) gives the same order as one band of
    all tile rows, and still visits every tile once."""
    M, N, K = 128, 4096 * 64, 64
    try:
        binding.set_config("BM=64,BN=64,WM=2,WN=2,G=1048576,XCD=1,KALT=0")
        big = binding.debug_schedule("matmul", M, N, K, 256)
        binding.set_config("BM=64,BN=64,WM=2,WN=2,G=2,XCD=1,KALT=0")
        two = binding.debug_schedule("matmul", M, N, K, 256)
    finally:
        binding.set_config(None)
    assert big == two
    assert len(big) == 2 * 4096
    assert {(tm, tn) for (_, _, tm, tn, _) in big} == {(i, j) for i in range(2) for j in range(4096)}


def test_c_program_uses_the_abi_without_a_gpu():
    """tests/c/mm_from_c.c: the header and library used from plain C11
    (argument errors, status strings, the configuration string)."""
    import subprocess
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "c"))
    import build_c_test
    exe = build_c_test.BIN if os.path.exists(build_c_test.BIN) else build_c_test.build()
    r = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
