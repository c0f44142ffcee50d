"""Race check: the library built with MM_DEBUG_FULL_SYNC (the slab kernel
drains every global->LDS copy and waits at a barrier before each super-step)
against the normal build, bit for bit.

The extra waits change only timing, never the arithmetic or its order, so any
difference means the normal build reads an LDS unit before its copy landed, or
overwrites one that a wave still reads.  (The pages trace a wrong result to a
missing write-after-read synchronisation in the pipelined K loop: PR
"Translate MmaOp patterns properly on Hopper", commit list.)  The cases cover
every slab instance: the four operand storages, the FFN fusion, the second
(pre-activation) output, chunk-major and stream-K split-K, and grids small
enough that the ring runs on across several tiles per workgroup; and the
skinny kernel's LDS ring (one and two activation blocks, unsplit and in
slices).
"""
import ctypes

import numpy as np
import pytest
import torch

from dense_bf16_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu

SLAB = "BM=256,BN=256,WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3"


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return binding.load(), binding.open_library(binding.FULLSYNC_LIB_PATH)


def say(*a):
    print("case:", *a, flush=True)


def stream():
    return torch.cuda.current_stream().cuda_stream


def assert_slab(libs, cfg, form, M, N, K, layout):
    """The configuration selects the slab kernel (the one these builds differ in)."""
    lib = libs[0]
    buf = ctypes.create_string_buffer(256)
    binding.check(lib.mm_set_config(cfg.encode() if cfg else None), "mm_set_config")
    try:
        binding.check(lib.mm_describe_config(1 if form == "ffn" else 0, M, N, K, binding.LAYOUTS[layout],
                                             buf, 256), "mm_describe_config")
    finally:
        binding.check(lib.mm_set_config(None), "mm_set_config")
    assert "KERNEL=gemm_nt_slab" in buf.value.decode(), buf.value.decode()


def run_both(libs, cfg, call, outs):
    """Runs `call(lib)` with each build under the same configuration and
    returns the outputs' bytes per build."""
    got = []
    for lib in libs:
        binding.check(lib.mm_set_config(cfg.encode() if cfg else None), "mm_set_config")
        try:
            for o in outs:
                o.view(torch.uint8).fill_(0xFF)
            call(lib)
            torch.cuda.synchronize()
            got.append([o.view(torch.uint8).cpu().numpy().copy() for o in outs])
        finally:
            binding.check(lib.mm_set_config(None), "mm_set_config")
    return got


def assert_same(got):
    (a, b) = got
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "the full-sync build differs from the normal build"


def operands(M, N, K, layout, seed, dev):
    a = synth.randn_bf16((M, K), 1.0, seed)
    b = synth.randn_bf16((K, N), K ** -0.5, seed + 1)
    A = a.t().contiguous() if layout[0] == "t" else a
    B = b.t().contiguous() if layout[1] == "t" else b
    return A.to(dev), B.to(dev)


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("grid", [0, 5])
def test_linear_and_matmul_all_storages(libs, layout, grid):
    dev = torch.device("cuda:0")
    M, N, K = 1040, 776, 1024  # 5 x 4 tiles (ragged), 16 super-steps
    cfg = SLAB + f",GRID={grid}"
    A, B = operands(M, N, K, layout, 900 + grid, dev)
    bias = synth.randn_bf16((N,), 1.0, 950).to(dev)
    lay = binding.LAYOUTS[layout]
    assert_slab(libs, cfg, "linear", M, N, K, layout)
    say("linear bias+GELU", layout, (M, N, K), cfg)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_linear(
        A.data_ptr(), B.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K, lay,
        binding.EPILOGUES["bias_gelu_tanh"], stream()), "mm_linear"), [out]))
    say("matmul f32", layout, (M, N, K), cfg)
    out32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_matmul(
        A.data_ptr(), B.data_ptr(), out32.data_ptr(), M, N, K, lay, 1, stream()), "mm_matmul"),
        [out32]))


@pytest.mark.parametrize("grid", [0, 7])
def test_ffn_and_preact(libs, grid):
    dev = torch.device("cuda:0")
    M, N, K = 776, 1160, 768
    x = synth.randn_bf16((M, K), 1.0, 960).to(dev)
    Wg = synth.randn_bf16((N, K), K ** -0.5, 961).to(dev)
    Wu = synth.randn_bf16((N, K), K ** -0.5, 962).to(dev)
    bias = synth.randn_bf16((N,), 1.0, 963).to(dev)
    cfg = f"BM=256,BN=256,WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3,GRID={grid}"
    assert_slab(libs, cfg, "ffn", M, N, K, "nt")
    assert_slab(libs, cfg, "linear", M, N, K, "nt")
    say("ffn swiglu", (M, N, K), cfg)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_ffn_swiglu(
        x.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), out.data_ptr(), M, N, K, stream()),
        "mm_ffn_swiglu"), [out]))
    say("linear with pre-activation", (M, N, K), cfg)
    pre = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_linear_preact(
        x.data_ptr(), Wg.data_ptr(), bias.data_ptr(), out.data_ptr(), pre.data_ptr(), M, N, K,
        binding.LAYOUTS["nt"], binding.EPILOGUES["bias_gelu_tanh"], stream()), "mm_linear_preact"),
        [out, pre]))


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("case", [(520, 392, 8192, None), (520, 392, 8200, None),
                                  (304, 264, 2048, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=3,GRID=6")])
def test_splitk(libs, layout, case):
    dev = torch.device("cuda:0")
    M, N, K, cfg = case
    A, B = operands(M, N, K, layout, 970, dev)
    lay = binding.LAYOUTS[layout]
    sizes = []
    for lib in libs:
        binding.check(lib.mm_set_config(cfg.encode() if cfg else None), "mm_set_config")
        n = ctypes.c_int64(0)
        binding.check(lib.mm_workspace_size(0, M, N, K, lay, ctypes.byref(n)), "mm_workspace_size")
        binding.check(lib.mm_set_config(None), "mm_set_config")
        sizes.append(n.value)
    assert sizes[0] == sizes[1] > 0, "this shape should take the split-K path"
    ws = torch.empty(sizes[0], dtype=torch.uint8, device=dev)
    say("split-K", layout, (M, N, K), cfg, sizes[0])
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_matmul_ws(
        A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, lay, 1, ws.data_ptr(), ws.numel(),
        stream()), "mm_matmul_ws"), [out]))


@pytest.mark.parametrize("grid", [0, 5])
def test_linear_bias_staged(libs, grid):
    """The instance that brings each tile's bias into LDS under the K loop
    (BSTAGE=1): ragged tiles load their bias in the epilogue, interior tiles
    read it from LDS."""
    dev = torch.device("cuda:0")
    M, N, K = 1040, 776, 1024
    cfg = SLAB + f",GRID={grid},BSTAGE=1"
    A, B = operands(M, N, K, "nt", 980 + grid, dev)
    bias = synth.randn_bf16((N,), 1.0, 985).to(dev)
    assert_slab(libs, cfg, "linear", M, N, K, "nt")
    for epi in ("bias", "bias_gelu_tanh"):
        say("linear, bias staged", epi, (M, N, K), cfg)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_linear(
            A.data_ptr(), B.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K,
            binding.LAYOUTS["nt"], binding.EPILOGUES[epi], stream()), "mm_linear"), [out]))


@pytest.mark.parametrize("bn", [192, 128])
@pytest.mark.parametrize("grid", [0, 5])
def test_linear_narrow_tiles(libs, bn, grid):
    """The 256 x 192 and 256 x 128 instances of the slab kernel (ragged tiles;
    on a grid of 5 the ring runs on across several tiles per workgroup)."""
    dev = torch.device("cuda:0")
    M, N, K = 1040, 776, 1024
    cfg = f"BM=256,BN={bn},WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3,GRID={grid}"
    A, B = operands(M, N, K, "nt", 990 + grid, dev)
    bias = synth.randn_bf16((N,), 1.0, 995).to(dev)
    assert_slab(libs, cfg, "linear", M, N, K, "nt")
    say("linear, narrow tiles", (M, N, K), cfg)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_linear(
        A.data_ptr(), B.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K,
        binding.LAYOUTS["nt"], binding.EPILOGUES["bias_gelu_tanh"], stream()), "mm_linear"), [out]))
    out32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_matmul(
        A.data_ptr(), B.data_ptr(), out32.data_ptr(), M, N, K, binding.LAYOUTS["nt"], 1, stream()),
        "mm_matmul"), [out32]))


@pytest.mark.parametrize("layout,bn", [("nt", 256), ("nt", 192), ("nt", 128), ("nn", 256), ("tn", 256),
                                       ("tt", 256)])
@pytest.mark.parametrize("grid", [0, 5])
def test_ragged_k(libs, layout, bn, grid):
    """The instances whose last super-step per tile is a partial one (K = 1000:
    15 whole super-steps and 40 k more; with K alternation half the tiles
    fetch the partial one first), in every operand storage."""
    dev = torch.device("cuda:0")
    M, N, K = 1040, 776, 1000
    cfg = f"BM=256,BN={bn},WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3,GRID={grid}"
    A, B = operands(M, N, K, layout, 1000 + grid, dev)
    bias = synth.randn_bf16((N,), 1.0, 1005).to(dev)
    assert_slab(libs, cfg, "linear", M, N, K, layout)
    say("linear, ragged K", layout, (M, N, K), cfg)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_linear(
        A.data_ptr(), B.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K,
        binding.LAYOUTS[layout], binding.EPILOGUES["bias_gelu_tanh"], stream()), "mm_linear"), [out]))


@pytest.mark.parametrize("grid", [0, 7])
def test_ffn_ragged_k(libs, grid):
    """The FFN's ragged-K instance (gate and up rows both masked past K)."""
    dev = torch.device("cuda:0")
    M, N, K = 776, 1160, 1000
    x = synth.randn_bf16((M, K), 1.0, 1010).to(dev)
    Wg = synth.randn_bf16((N, K), K ** -0.5, 1011).to(dev)
    Wu = synth.randn_bf16((N, K), K ** -0.5, 1012).to(dev)
    cfg = f"BM=256,BN=256,WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3,GRID={grid}"
    assert_slab(libs, cfg, "ffn", M, N, K, "nt")
    say("ffn swiglu, ragged K", (M, N, K), cfg)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, cfg, lambda lib: binding.check(lib.mm_ffn_swiglu(
        x.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), out.data_ptr(), M, N, K, stream()),
        "mm_ffn_swiglu"), [out]))


@pytest.mark.parametrize("case", [(16, 4104, 2056, True), (7, 1000, 8200, False), (7, 1000, 8200, True),
                                  (29, 2056, 4104, True), (32, 8192, 1032, False)])
def test_skinny(libs, case):
    """The skinny kernel's ring of LDS stages: the race-check build drains
    every copy before a stage is read and waits for every wave before the
    next copy is issued."""
    dev = torch.device("cuda:0")
    M, N, K, ws = case
    assert binding.describe_config("linear", M, N, K).endswith("KERNEL=gemm_skinny")
    A, B = operands(M, N, K, "nt", 990 + M, dev)
    bias = synth.randn_bf16((N,), 1.0, 991).to(dev)
    nbytes = binding.workspace_size("linear", M, N, K) if ws else 0
    assert nbytes > 0 or not ws, "this shape should be cut into slices"
    wsp = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    say("skinny", (M, N, K), "ws" if ws else "no ws", nbytes)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert_same(run_both(libs, None, lambda lib: binding.check(lib.mm_linear_ws(
        A.data_ptr(), B.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K, binding.LAYOUTS["nt"],
        binding.EPILOGUES["bias_gelu_tanh"], wsp.data_ptr() if ws else None, nbytes, stream()),
        "mm_linear_ws"), [out]))
