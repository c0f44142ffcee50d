"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* Index mapping, bit for bit: integer operands whose fp32 sums are exact in
  any order, every layout, every tile configuration, shapes that span
  several tiles with ragged M, N and K tails.
* Numerics at every workload's real size and launch configuration (the
  heuristic and automatic split-K, exactly as the benchmark runs them):
  every output element against the oracle's full output; bf16 outputs within
  2e-2*(|ref|+1), fp32 outputs within 1e-3*(|ref|+1).
* Index mapping at the same real shapes, storages and launches, bit for bit
  over the whole output, with integer operands.
* Edge cases: empty outputs, 1x1, unaligned fp32 rows, an output pointer
  that is not 16-byte aligned, guard bands around the output, repeatability,
  and an operand with more than 2^31 elements.
"""

import numpy as np
import pytest
import torch

import oracle
from dense_bf16_gemm_amd import binding, synth
import dense_bf16_gemm_amd as mm

pytestmark = pytest.mark.gpu

CONFIGS = [
    "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,PIPE=3",
    # a small persistent grid: several tiles per workgroup, K direction
    # alternating between them, prefetch running across tile boundaries
    "BM=256,BN=256,WM=2,WN=2,G=2,XCD=0,KALT=1,GRID=3,PIPE=3",
    "BM=256,BN=256,WM=2,WN=4,G=8,XCD=1,KALT=2,PIPE=2",
    "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,PIPE=1",
    # wave-specialized producer/consumer kernel (256 x 128 tiles), and with a
    # small grid so that the ring runs across several tiles per workgroup
    "BM=256,BN=128,WM=2,WN=4,G=8,XCD=1,KALT=2,PIPE=4",
    "BM=256,BN=128,WM=2,WN=4,G=2,XCD=0,KALT=2,GRID=3,PIPE=4",
    # two-group ping-pong over alternate 256 x 128 tiles; with a small grid
    # each workgroup swaps roles across many tiles, its epilogues running in
    # row blocks (K >= 8 super-steps) or whole (shorter K) under the other
    # group's K loop
    "BM=256,BN=128,WM=2,WN=4,G=8,XCD=1,KALT=2,PIPE=5",
    "BM=256,BN=128,WM=2,WN=4,G=2,XCD=0,KALT=2,GRID=3,PIPE=5",
    "BM=128,BN=128,WM=2,WN=2,G=4,XCD=1,KALT=1",
    "BM=64,BN=64,WM=2,WN=2,G=3,XCD=0,KALT=0",
    # 256 x 192 tiles (K-contiguous single-weight products; other layouts
    # and forms fall back to 256 x 256), also on a small grid
    "BM=256,BN=192,WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3",
    "BM=256,BN=192,WM=2,WN=2,G=2,XCD=0,KALT=1,GRID=3,PIPE=3",
    # 256 x 128 slab tiles (the same restriction), also on a small grid
    "BM=256,BN=128,WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3",
    "BM=256,BN=128,WM=2,WN=2,G=2,XCD=0,KALT=1,GRID=3,PIPE=3",
    # 64 x 64 tiles: K <= 256 runs the kernel holding all of K in LDS (here
    # on a small grid, several tiles per workgroup); PIPE=0 keeps the basic
    # two-stage kernel at every K
    "BM=64,BN=64,WM=2,WN=2,G=3,XCD=0,KALT=0,GRID=3",
    "BM=64,BN=64,WM=2,WN=2,G=3,XCD=0,KALT=0,PIPE=0",
    # the slab instance that brings each tile's bias into LDS under the K
    # loop (bias epilogues of K-contiguous shapes with whole super-steps),
    # on a small grid so that the staging runs across several tiles
    "BM=256,BN=256,WM=2,WN=2,G=2,XCD=0,KALT=1,GRID=3,PIPE=3,BSTAGE=1",
]
FFN_CONFIGS = [
    "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,PIPE=3",
    # a small persistent grid: several tiles per workgroup, K direction
    # alternating between them, prefetch running across tile boundaries
    "BM=256,BN=256,WM=2,WN=2,G=2,XCD=0,KALT=1,GRID=3,PIPE=3",
    "BM=256,BN=256,WM=2,WN=4,G=8,XCD=1,KALT=2,PIPE=2",
    "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,PIPE=1",
    "BM=128,BN=256,WM=2,WN=2,G=4,XCD=1,KALT=1",
    "BM=128,BN=128,WM=2,WN=2,G=2,XCD=0,KALT=0",
]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _restore_config():
    yield
    binding.set_config(None)


def say(*a):
    print("case:", *a, flush=True)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def stream():
    return torch.cuda.current_stream().cuda_stream


def tol_excess(got: np.ndarray, ref: np.ndarray, rel: float) -> float:
    """max(|got - ref| - rel*(|ref| + 1)); <= 0 means within tolerance."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref) - rel * (np.abs(ref) + 1.0)))


def call_linear(A, B, bias, M, N, K, layout, epi, out):
    lib = binding.load()
    st = lib.mm_linear(A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None,
                       out.data_ptr(), M, N, K, binding.LAYOUTS[layout], binding.EPILOGUES[epi],
                       stream())
    binding.check(st, "mm_linear")


def call_matmul(A, B, M, N, K, layout, out_f32, out):
    lib = binding.load()
    st = lib.mm_matmul(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, binding.LAYOUTS[layout],
                       1 if out_f32 else 0, stream())
    binding.check(st, "mm_matmul")


def call_ffn(x, Wg, Wu, M, N, K, act, out):
    lib = binding.load()
    st = lib.mm_ffn_glu(x.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), out.data_ptr(), M, N, K,
                        binding.GLU_ACTS[act], stream())
    binding.check(st, "mm_ffn_glu")


# ------------------------------------------------------------ index mapping
def shapes_for(layout):
    """(M, N, K) spanning several tiles with ragged tails; contiguous extents
    stay multiples of 8 as the ABI requires (A's rows are M long for TN/TT,
    B's rows are N long for NN/TN)."""
    # the last three have K a multiple of 64 (>= 128), the whole-line slab
    # kernel's domain; the others take the 32-k pipeline or the basic kernel
    base = [(1, 8, 8), (17, 24, 72), (129, 136, 64), (300, 264, 200), (520, 392, 4104),
            (257, 520, 128), (300, 264, 192), (520, 392, 4160)]
    out = []
    for M, N, K in base:
        if layout in ("tn", "tt"):
            M = -(-M // 8) * 8
        if layout in ("nt", "tt"):
            N = N + 3
        out.append((M, N, K))
    return out


def test_ws_config_selects_ws_kernel():
    """PIPE=4 runs the wave-specialized kernel where it applies and the default
    slab tile elsewhere (a partial last super-step, FFN), the 32-k pipeline
    below two super-steps."""
    binding.set_config("BM=256,BN=128,WM=2,WN=4,G=8,XCD=1,KALT=2,PIPE=4")
    try:
        for (M, N, K) in shapes_for("nt")[-3:]:
            assert binding.describe_config("linear", M, N, K).endswith("KERNEL=gemm_ws")
        assert binding.describe_config("linear", 300, 267, 200).endswith("KERNEL=gemm_nt_slab")
        assert binding.describe_config("linear", 300, 267, 72).endswith("KERNEL=gemm_nt_pipe")
        assert binding.describe_config("ffn", 300, 515, 256).endswith("KERNEL=gemm_nt_slab")
    finally:
        binding.set_config(None)


def test_pp_config_selects_pp_kernel():
    """PIPE=5 runs the ping-pong kernel where it applies (K-contiguous single
    weight, whole super-steps) and the default slab tile elsewhere."""
    binding.set_config("BM=256,BN=128,WM=2,WN=4,G=8,XCD=1,KALT=2,PIPE=5")
    try:
        for (M, N, K) in shapes_for("nt")[-3:]:
            assert binding.describe_config("linear", M, N, K).endswith("KERNEL=gemm_pp")
        assert binding.describe_config("linear", 300, 267, 200).endswith("KERNEL=gemm_nt_slab")
        assert binding.describe_config("linear", 300, 267, 72).endswith("KERNEL=gemm_nt_pipe")
        assert binding.describe_config("ffn", 300, 515, 256).endswith("KERNEL=gemm_nt_slab")
        assert binding.describe_config("matmul", 520, 392, 4160, "nn").endswith("KERNEL=gemm_nt_slab")
    finally:
        binding.set_config(None)


def test_slab_shapes_select_slab_kernel():
    binding.set_config(CONFIGS[0])
    try:
        for (M, N, K) in shapes_for("nt")[-3:]:
            assert binding.describe_config("linear", M, N, K).endswith("KERNEL=gemm_nt_slab")
        assert binding.describe_config("ffn", 300, 515, 256).endswith("KERNEL=gemm_nt_slab")
    finally:
        binding.set_config(None)


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt"])
def test_mapping_bitexact_linear_bias(dev, cfg, layout):
    binding.set_config(cfg)
    for (M, N, K) in shapes_for(layout):
        say("mapping linear+bias", layout, cfg, (M, N, K))
        ops = synth.mapping_operands(M, N, K, layout, seed=M * 7 + N * 3 + K, with_bias=True)
        A, B, bias = ops["A"], ops["B"], ops["bias"]
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        call_linear(A.to(dev), B.to(dev), bias.to(dev), M, N, K, layout, "bias", out)
        torch.cuda.synchronize()
        _, ref_bits = oracle.gemm(synth.bits(A), synth.bits(B), layout, "bias", bias=synth.bits(bias))
        got = to_bits(out)
        bad = np.argwhere(got != ref_bits)
        assert bad.size == 0, f"{layout} {cfg} {(M, N, K)}: {len(bad)} mismatches, first {bad[:5].tolist()}"


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt"])
def test_mapping_bitexact_matmul_f32(dev, cfg, layout):
    binding.set_config(cfg)
    for (M, N, K) in shapes_for(layout)[:4] + [(264, 136, 2056), (264, 136, 2112)]:
        say("mapping matmul f32", layout, cfg, (M, N, K))
        A, B = synth.dense_int_operands(M, N, K, layout, seed=M + N + K)
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
        call_matmul(A.to(dev), B.to(dev), M, N, K, layout, True, out)
        torch.cuda.synchronize()
        ref, _ = oracle.gemm(synth.bits(A), synth.bits(B), layout)
        np.testing.assert_array_equal(out.cpu().numpy(), ref)


# ------------------------------------------------------------ batched forms
def call_matmul_batched(A, B, batch, M, N, K, sa, sb, so, layout, out_f32, out):
    lib = binding.load()
    st = lib.mm_matmul_batched(A.data_ptr(), B.data_ptr(), out.data_ptr(), batch, M, N, K, sa, sb, so,
                               binding.LAYOUTS[layout], 1 if out_f32 else 0, stream())
    binding.check(st, "mm_matmul_batched")


# (batch, M, N, K, layout, B broadcast): K multiples of 64 with NT take the
# slab kernel, the rest the basic kernel (the batched form runs on those two)
BATCH_CASES = [
    (3, 129, 136, 200, "nt", False),
    (2, 300, 264, 192, "nt", False),
    (3, 257, 520, 128, "nt", True),
    (4, 64, 72, 128, "nn", False),
    (2, 136, 200, 72, "tn", True),
    (2, 136, 208, 64, "tt", False),
]


@pytest.mark.parametrize("case", range(len(BATCH_CASES)))
@pytest.mark.parametrize("out_f32", [True, False])
def test_batched_mapping_bitexact(dev, case, out_f32):
    batch, M, N, K, layout, bcast = BATCH_CASES[case]
    say("batched mapping", BATCH_CASES[case], "f32" if out_f32 else "bf16")
    As, Bs = [], []
    for b in range(batch):
        A, B = synth.dense_int_operands(M, N, K, layout, seed=100 * b + M + N + K)
        As.append(A)
        Bs.append(Bs[0] if (bcast and b) else B)
    A_all = torch.stack(As).to(dev)
    B_all = (Bs[0].unsqueeze(0) if bcast else torch.stack(Bs)).to(dev)
    sa = As[0].numel()
    sb = 0 if bcast else Bs[0].numel()
    out = torch.full((batch, M, N), float("nan"), dtype=torch.float32 if out_f32 else torch.bfloat16,
                     device=dev)
    call_matmul_batched(A_all, B_all, batch, M, N, K, sa, sb, M * N, layout, out_f32, out)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, bits = oracle.gemm(synth.bits(As[b]), synth.bits(Bs[b]), layout)
        if out_f32:
            np.testing.assert_array_equal(out[b].cpu().numpy(), ref)
        else:
            np.testing.assert_array_equal(to_bits(out[b]), bits)


def test_batched_torch_views_and_linear(dev):
    """mm.bmm on torch views (a transposed batch, a broadcast entry) and the
    batched linear layer with a shared weight and bias + GELU."""
    batch, M, N, K = 3, 200, 264, 256
    say("batched views + linear", (batch, M, N, K))
    A = synth.randn_bf16((batch, M, K), 1.0, 21).to(dev)
    Bt = synth.randn_bf16((batch, N, K), K ** -0.5, 22).to(dev)
    got = mm.bmm(A, Bt.transpose(1, 2), torch.float32)
    torch.cuda.synchronize()
    for b in range(batch):
        y, _ = oracle.gemm(synth.bits(A[b].cpu()), synth.bits(Bt[b].cpu()), "nt")
        assert tol_excess(got[b].cpu().numpy(), y, 1e-3) <= 0
    W = synth.randn_bf16((N, K), K ** -0.5, 23).to(dev)
    bias = synth.randn_bf16((N,), 1.0, 24).to(dev)
    got = mm.linear_batched(A, W, bias, "bias_gelu_tanh")
    torch.cuda.synchronize()
    for b in range(batch):
        y, _ = oracle.gemm(synth.bits(A[b].cpu()), synth.bits(W.cpu()), "nt", "bias_gelu_tanh",
                           bias=synth.bits(bias.cpu()))
        assert tol_excess(got[b].float().cpu().numpy(), y, 2e-2) <= 0
    # a broadcast activation entry (expand gives stride 0) against per-entry weights
    got = mm.bmm(A[:1].expand(batch, M, K), Bt.transpose(1, 2), torch.float32)
    torch.cuda.synchronize()
    for b in range(batch):
        y, _ = oracle.gemm(synth.bits(A[0].cpu()), synth.bits(Bt[b].cpu()), "nt")
        assert tol_excess(got[b].cpu().numpy(), y, 1e-3) <= 0


# ------------------------------------------------------------ split-K
# (M, N, K, configuration): few 256 x 256 output tiles, long K.  The forced
# slice counts with small grids make slices wait on other workgroups across
# rounds of work units.
# ------------------------------------------------ two outputs: GELU and its input
def call_linear_preact(A, B, bias, M, N, K, layout, epi, out, pre):
    lib = binding.load()
    st = lib.mm_linear_preact(A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None,
                              out.data_ptr(), pre.data_ptr(), M, N, K, binding.LAYOUTS[layout],
                              binding.EPILOGUES[epi], stream())
    binding.check(st, "mm_linear_preact")


# (M, N, K, layout): slab kernel (interior and edge tiles), ragged K and the
# [K][N] weight layout (basic kernel)
PREACT_CASES = [(512, 512, 256, "nt"), (300, 267, 192, "nt"), (257, 139, 200, "nt"),
                (129, 136, 72, "nn"), (520, 392, 4160, "nt")]


@pytest.mark.parametrize("case", range(len(PREACT_CASES)))
def test_preact_mapping_bitexact(dev, case):
    """Integer operands: the pre-activation (bias included) is exact in fp32
    and bf16, so it must match the oracle's bias epilogue bit for bit; the
    GELU output is checked against the oracle's bias+GELU within 2e-2."""
    M, N, K, layout = PREACT_CASES[case]
    say("preact mapping", PREACT_CASES[case])
    ops = synth.mapping_operands(M, N, K, layout, seed=M + 5 * N + K, with_bias=True)
    A, B, bias = ops["A"], ops["B"], ops["bias"]
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    pre = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    call_linear_preact(A.to(dev), B.to(dev), bias.to(dev), M, N, K, layout, "bias_gelu_tanh", out, pre)
    torch.cuda.synchronize()
    _, pre_bits = oracle.gemm(synth.bits(A), synth.bits(B), layout, "bias", bias=synth.bits(bias))
    np.testing.assert_array_equal(to_bits(pre), pre_bits)
    y, _ = oracle.gemm(synth.bits(A), synth.bits(B), layout, "bias_gelu_tanh", bias=synth.bits(bias))
    assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0


@pytest.mark.parametrize("epi", ["gelu_tanh", "bias_gelu_tanh"])
def test_preact_random_matches_single_output(dev, epi):
    """Seeded normal data: both outputs within tolerance of the oracle, and
    bit-identical to the single-output calls (same kernel arithmetic)."""
    M, N, K = 520, 392, 512
    say("preact random", epi, (M, N, K))
    x = synth.randn_bf16((M, K), 1.0, 31).to(dev)
    W = synth.randn_bf16((N, K), K ** -0.5, 32).to(dev)
    bias = synth.randn_bf16((N,), 1.0, 33).to(dev) if epi == "bias_gelu_tanh" else None
    out, pre = mm.linear_preact(x, W, bias, epi)
    one = mm.linear(x, W, bias, epi)
    pre_one = mm.linear(x, W, bias, "bias" if bias is not None else "none", workspace=None)
    torch.cuda.synchronize()
    bb = synth.bits(bias.cpu()) if bias is not None else None
    y, _ = oracle.gemm(synth.bits(x.cpu()), synth.bits(W.cpu()), "nt", epi, bias=bb)
    t, _ = oracle.gemm(synth.bits(x.cpu()), synth.bits(W.cpu()), "nt", "bias" if bb is not None else "none",
                       bias=bb)
    assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0
    assert tol_excess(pre.float().cpu().numpy(), t, 2e-2) <= 0
    assert torch.equal(out.view(torch.int16), one.view(torch.int16))
    assert torch.equal(pre.view(torch.int16), pre_one.view(torch.int16))


# (M, N, K, config): automatic chunk-major (the cost model's chunk count and
# tile width, one chunk per workgroup); forced stream-K on 140 tiles (ranges
# of 3/4 of a tile);
# ranges of two chunks of three that cross tile boundaries; ranges of
# three of four; uneven chunk-major chunks (64 super-steps in 7); and K not a
# multiple of 64 (the last chunk of each tile ends with a partial super-step),
# chunk-major and in stream-K ranges
SK_CASES = [
    (520, 395, 8192, None),
    (520, 395, 8200, None),
    (300, 264, 2056, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=3,GRID=6"),
    (2560, 3584, 2048, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=4"),
    (300, 264, 2048, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=3,GRID=6"),
    (257, 520, 1024, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=0,KALT=2,SK=4,GRID=10"),
    (64, 8, 4096, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=7"),
]


def call_matmul_ws(A, B, M, N, K, out_f32, out, ws, nbytes):
    lib = binding.load()
    st = lib.mm_matmul_ws(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, binding.LAYOUTS["nt"],
                          1 if out_f32 else 0, ws.data_ptr() if ws is not None else None, nbytes,
                          stream())
    binding.check(st, "mm_matmul_ws")


@pytest.mark.parametrize("case", range(len(SK_CASES)))
@pytest.mark.parametrize("out_f32", [True, False])
def test_splitk_mapping_bitexact(dev, case, out_f32):
    """Integer operands keep every partial sum exact, so the slices' sums,
    added in any order, must give the oracle's bits."""
    M, N, K, cfg = SK_CASES[case]
    binding.set_config(cfg)
    try:
        nbytes = binding.workspace_size("matmul", M, N, K)
        say("split-K mapping", (M, N, K), cfg, "f32" if out_f32 else "bf16", nbytes)
        assert nbytes > 0, "this shape should take the split-K path"
        # stale contents must not matter: the workspace starts as NaN bytes
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
        A, B = synth.dense_int_operands(M, N, K, "nt", seed=M + 3 * N + K)
        A, B = A.to(dev), B.to(dev)
        ref, bits = oracle.gemm(synth.bits(A.cpu()), synth.bits(B.cpu()), "nt")
        out = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dev)
        for rep in range(3):  # the same workspace again
            out.fill_(float("nan"))
            call_matmul_ws(A, B, M, N, K, out_f32, out, ws, nbytes)
            torch.cuda.synchronize()
            if out_f32:
                np.testing.assert_array_equal(out.cpu().numpy(), ref)
            else:
                np.testing.assert_array_equal(to_bits(out), bits)
    finally:
        binding.set_config(None)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("case", [(520, 392, 8192, None), (520, 392, 8200, None),
                                  (304, 264, 2048, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=3,GRID=6")])
def test_splitk_mapping_layouts(dev, layout, case):
    """Split-K (chunk-major, and stream-K ranges across tile boundaries) with
    operands stored [K][M] / [K][N]: integer operands, the oracle's bits."""
    M, N, K, cfg = case
    binding.set_config(cfg)
    try:
        nbytes = binding.workspace_size("matmul", M, N, K, layout)
        say("split-K layouts", layout, (M, N, K), cfg, nbytes)
        assert nbytes > 0, "this shape should take the split-K path"
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
        A, B = synth.dense_int_operands(M, N, K, layout, seed=M + 5 * N + K)
        ref, bits = oracle.gemm(synth.bits(A), synth.bits(B), layout)
        Ad, Bd = A.to(dev), B.to(dev)  # held for the whole call
        lib = binding.load()
        for out_f32 in (True, False):
            out = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dev)
            st = lib.mm_matmul_ws(Ad.data_ptr(), Bd.data_ptr(), out.data_ptr(), M, N, K,
                                  binding.LAYOUTS[layout], 1 if out_f32 else 0, ws.data_ptr(), nbytes, stream())
            binding.check(st, "mm_matmul_ws")
            torch.cuda.synchronize()
            if out_f32:
                np.testing.assert_array_equal(out.cpu().numpy(), ref)
            else:
                np.testing.assert_array_equal(to_bits(out), bits)
    finally:
        binding.set_config(None)


def test_splitk_workspace_shared_across_shapes(dev):
    """One workspace, calls of two shapes with different workgroup counts and
    dealings alternating (chunk-major 16 chunks on 6 tiles; stream-K ranges on
    4 tiles): each call reads only the slots it has just written, so every
    result keeps the oracle's bits."""
    cases = [(520, 395, 8192, None), (300, 264, 2048, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=3,GRID=6")]
    sizes = []
    for (M, N, K, cfg) in cases:
        binding.set_config(cfg)
        sizes.append(binding.workspace_size("matmul", M, N, K))
    binding.set_config(None)
    assert min(sizes) > 0
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device=dev)
    ops = []
    for (M, N, K, cfg) in cases:
        A, B = synth.dense_int_operands(M, N, K, "nt", seed=7 * M + N + K)
        _, bits = oracle.gemm(synth.bits(A), synth.bits(B), "nt")
        ops.append((A.to(dev), B.to(dev), bits))
    for rep in range(3):
        for (M, N, K, cfg), (A, B, bits) in zip(cases, ops):
            say("shared workspace", rep, (M, N, K), cfg)
            binding.set_config(cfg)
            try:
                out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                call_matmul_ws(A, B, M, N, K, False, out, ws, ws.numel())
                torch.cuda.synchronize()
            finally:
                binding.set_config(None)
            np.testing.assert_array_equal(to_bits(out), bits)


def test_splitk_auto_workspace_two_streams(dev):
    """workspace="auto" keeps one workspace per stream: split-K calls of two
    shapes in flight on two streams at once, with no synchronisation between
    the streams, each keep the oracle's bits."""
    from dense_bf16_gemm_amd import gemm as gemm_mod
    cases = [(520, 395, 8192), (300, 650, 8192)]
    for (M, N, K) in cases:
        assert binding.workspace_size("matmul", M, N, K) > 0, "these shapes should take the split-K path"
    ops = []
    for (M, N, K) in cases:
        A, Bt = synth.dense_int_operands(M, N, K, "nt", seed=11 * M + N + K)
        _, bits = oracle.gemm(synth.bits(A), synth.bits(Bt), "nt")
        ops.append((A.to(dev), Bt.to(dev), bits))
    streams = [torch.cuda.Stream(device=dev) for _ in cases]
    keys = [(dev.index, s.cuda_stream) for s in streams]
    outs = [[] for _ in cases]
    try:
        for s in streams:  # the operands were written on the current stream
            s.wait_stream(torch.cuda.current_stream(dev))
        for rep in range(4):
            for i, ((M, N, K), (A, Bt, _), s) in enumerate(zip(cases, ops, streams)):
                say("auto workspace, two streams", rep, i, (M, N, K))
                with torch.cuda.stream(s):
                    outs[i].append(mm.matmul(A, Bt.t()))
        torch.cuda.synchronize()
        assert set(keys) <= set(gemm_mod._workspaces), "each stream keeps its own workspace"
        assert len({gemm_mod._workspaces[k].data_ptr() for k in keys}) == len(keys)
        for (_, _, bits), got in zip(ops, outs):
            for out in got:
                np.testing.assert_array_equal(to_bits(out), bits)
    finally:
        torch.cuda.synchronize()
        mm.release_workspaces(dev)
        assert not any(k[0] == dev.index for k in gemm_mod._workspaces)


@pytest.mark.parametrize("case", [(520, 395, 8192, None), (520, 395, 8200, None),
                                  (304, 264, 2048, "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=3,GRID=6")])
def test_splitk_linear_epilogues(dev, case):
    """Split-K of the linear form: the reduction adds the pieces in k order,
    then applies the bias and GELU once.  Integer operands and bias keep the
    bias epilogue bit-exact; the GELU epilogues (random operands) stay within
    the bf16 tolerance; chunk-major and stream-K dealings, ragged tiles."""
    M, N, K, cfg = case
    binding.set_config(cfg)
    try:
        nbytes = binding.workspace_size("linear", M, N, K)
        say("split-K linear", (M, N, K), cfg, nbytes)
        assert nbytes > 0, "this shape should take the split-K path"
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
        ops = synth.mapping_operands(M, N, K, "nt", seed=M + 9 * N + K, with_bias=True)
        x, W, bias = ops["A"].to(dev), ops["B"].to(dev), ops["bias"].to(dev)
        out = mm.linear(x, W, bias, "bias", workspace=ws)
        torch.cuda.synchronize()
        _, bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), "nt", "bias",
                              bias=synth.bits(ops["bias"]))
        np.testing.assert_array_equal(to_bits(out), bits)
        x = synth.randn_bf16((M, K), 1.0, 41)
        W = synth.randn_bf16((N, K), K ** -0.5, 42)
        b = synth.randn_bf16((N,), 1.0, 43)
        for epi in ("gelu_tanh", "bias_gelu_tanh"):
            out = mm.linear(x.to(dev), W.to(dev), b.to(dev) if "bias" in epi else None, epi, workspace=ws)
            torch.cuda.synchronize()
            y, _ = oracle.gemm(synth.bits(x), synth.bits(W), "nt", epi,
                               bias=synth.bits(b) if "bias" in epi else None)
            assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0, epi
    finally:
        binding.set_config(None)


def test_splitk_random_and_fallbacks(dev):
    M, N, K = 700, 900, 16384
    x = synth.randn_bf16((M, K), 1.0, 11).to(dev)
    W = synth.randn_bf16((N, K), 2.0 ** -7, 12).to(dev)
    say("split-K random", (M, N, K))
    nbytes = binding.workspace_size("matmul", M, N, K)
    assert nbytes > 0
    y, _ = oracle.gemm(synth.bits(x.cpu()), synth.bits(W.cpu()), "nt")
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    call_matmul_ws(x, W.t(), M, N, K, True, out, ws, nbytes)
    torch.cuda.synchronize()
    assert tol_excess(out.cpu().numpy(), y, 1e-3) <= 0
    # run to run identical (slices are added in a fixed order)
    out2 = torch.empty_like(out)
    call_matmul_ws(x, W.t(), M, N, K, True, out2, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    # no workspace: the unsplit kernel, same tolerance
    out3 = torch.empty_like(out)
    call_matmul_ws(x, W.t(), M, N, K, True, out3, None, 0)
    torch.cuda.synchronize()
    assert tol_excess(out3.cpu().numpy(), y, 1e-3) <= 0
    # linear with epilogue "none" takes the same path (bf16 out)
    got = mm.linear(x, W, None, "none")
    torch.cuda.synchronize()
    assert tol_excess(got.float().cpu().numpy(), y, 2e-2) <= 0
    # a workspace smaller than reported is refused before any launch
    with pytest.raises(binding.MMError) as e:
        call_matmul_ws(x, W.t(), M, N, K, True, out3, ws, nbytes - 256)
    assert e.value.status == binding.MM_ERR_INVALID_VALUE
    # a workspace overlapping the output is refused
    with pytest.raises(binding.MMError) as e:
        call_matmul_ws(x, W.t(), M, N, K, True, out3, out3.view(torch.uint8), out3.numel() * 4)
    assert e.value.status == binding.MM_ERR_INVALID_VALUE


@pytest.mark.parametrize("cfg", FFN_CONFIGS)
def test_mapping_bitexact_ffn(dev, cfg):
    binding.set_config(cfg)
    for (M, N, K) in [(1, 3, 8), (130, 200, 72), (300, 515, 264), (520, 264, 1032), (300, 515, 256),
                      (520, 264, 1088)]:
        say("mapping ffn glu_identity", cfg, (M, N, K))
        ops = synth.mapping_operands(M, N, K, "nt", seed=M + 5 * N + K, gated=True)
        x, Wg, Wu = ops["A"], ops["B"], ops["B2"]
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        call_ffn(x.to(dev), Wg.to(dev), Wu.to(dev), M, N, K, "identity", out)
        torch.cuda.synchronize()
        _, ref_bits = oracle.gemm(synth.bits(x), synth.bits(Wg), "nt", "glu_identity", B2=synth.bits(Wu))
        got = to_bits(out)
        bad = np.argwhere(got != ref_bits)
        assert bad.size == 0, f"ffn {cfg} {(M, N, K)}: {len(bad)} mismatches, first {bad[:5].tolist()}"


# ------------------------------------------------------------ numerics
@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("epi", ["none", "bias", "gelu_tanh", "bias_gelu_tanh"])
@pytest.mark.parametrize("K", [520, 512])
def test_linear_epilogues_random(dev, cfg, epi, K):
    binding.set_config(cfg)
    M, N = 333, 270
    say("linear random", epi, cfg)
    x = synth.randn_bf16((M, K), 1.0, 1)
    W = synth.randn_bf16((N, K), K ** -0.5, 2)
    b = synth.randn_bf16((N,), 1.0, 3)
    out = mm.linear(x.to(dev), W.to(dev), b.to(dev), epi)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(x), synth.bits(W), "nt", epi, bias=synth.bits(b))
    assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("epi", ["bias_gelu_tanh", "none"])
def test_transposed_storage_random(dev, layout, epi):
    """Operands stored [K][M] / [K][N] (the slab kernel's transpose-read forms
    at K a multiple of 64, several tiles, ragged M and N), N(0,1) data, against
    the oracle within the bf16 and fp32 tolerances."""
    M, N, K = 520, 392, 512
    say("transposed storage random", layout, epi, (M, N, K))
    a_shape = (K, M) if layout in ("tn", "tt") else (M, K)
    b_shape = (N, K) if layout in ("nt", "tt") else (K, N)
    A = synth.randn_bf16(a_shape, 1.0, 41)
    B = synth.randn_bf16(b_shape, K ** -0.5, 42)
    bias = synth.randn_bf16((N,), 1.0, 43)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    call_linear(A.to(dev), B.to(dev), bias.to(dev) if "bias" in epi else None, M, N, K, layout, epi, out)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(A), synth.bits(B), layout, epi,
                       bias=synth.bits(bias) if "bias" in epi else None)
    assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0
    out32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    call_matmul(A.to(dev), B.to(dev), M, N, K, layout, True, out32)
    torch.cuda.synchronize()
    y32, _ = oracle.gemm(synth.bits(A), synth.bits(B), layout)
    assert tol_excess(out32.cpu().numpy(), y32, 1e-3) <= 0


@pytest.mark.parametrize("cfg", FFN_CONFIGS)
@pytest.mark.parametrize("K", [264, 256])
def test_ffn_swiglu_random(dev, cfg, K):
    binding.set_config(cfg)
    M, N = 300, 390
    say("ffn swiglu random", cfg)
    x = synth.randn_bf16((M, K), 1.0, 4)
    Wg = synth.randn_bf16((N, K), K ** -0.5, 5)
    Wu = synth.randn_bf16((N, K), K ** -0.5, 6)
    out = mm.ffn_swiglu(x.to(dev), Wg.to(dev), Wu.to(dev))
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(x), synth.bits(Wg), "nt", "swiglu", B2=synth.bits(Wu))
    assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0


GUARD_BYTES = 4096


def guarded_out(M, N, f32, dev):
    """An [M, N] output inside a buffer with 4 KiB guard bands of NaN bytes
    on both sides (the output itself starts 4 KiB in: 16-byte aligned)."""
    esize = 4 if f32 else 2
    g = GUARD_BYTES // esize
    buf = torch.full((M * N + 2 * g,), float("nan"), dtype=torch.float32 if f32 else torch.bfloat16,
                     device=dev)
    return buf, buf[g:g + M * N].view(M, N)


def guards_intact(buf, M, N):
    g = GUARD_BYTES // buf.element_size()
    return bool(torch.isnan(buf[:g]).all()) and bool(torch.isnan(buf[g + M * N:]).all())


def run_workload(w: synth.Workload, t, dev, out=None):
    """One call of the workload exactly as bench.py makes it (the heuristic's
    configuration, split-K through the automatic workspace where it applies)."""
    g = {k: v.to(dev) for k, v in t.items()}
    if w.form == "matmul":
        A = g["A"] if "A" in g else g["At"].t()  # transposed views, read in place
        B = g["B"] if "B" in g else g["Bt"].t()
        return mm.matmul(A, B, torch.float32 if w.out_dtype == "f32" else torch.bfloat16, out=out)
    if w.form == "linear":
        return mm.linear(g["x"], g["W"], g["bias"], w.epilogue, out=out)
    return mm.ffn_swiglu(g["x"], g["W_gate"], g["W_up"], out=out)


def oracle_args(w: synth.Workload, t):
    if w.form == "matmul":
        A = t["A"] if "A" in t else t["At"]
        B = t["B"] if "B" in t else t["Bt"]
        return dict(A=synth.bits(A), B=synth.bits(B), layout=w.layout, epilogue="none")
    if w.form == "linear":
        return dict(A=synth.bits(t["x"]), B=synth.bits(t["W"]), layout="nt", epilogue=w.epilogue,
                    bias=synth.bits(t["bias"]))
    return dict(A=synth.bits(t["x"]), B=synth.bits(t["W_gate"]), B2=synth.bits(t["W_up"]),
                layout="nt", epilogue="swiglu")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity(dev, name):
    """Every output element of every workload at its real size, in the launch
    configuration bench.py times, against the oracle's full output; the 4 KiB
    around the output stay untouched."""
    w = synth.WORKLOADS[name]
    say("workload", name, binding.describe_config(w.form, w.M, w.N, w.K, w.layout))
    t = w.make()
    f32 = w.out_dtype == "f32"
    buf, out = guarded_out(w.M, w.N, f32, dev)
    run_workload(w, t, dev, out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, w.M, w.N)
    got = out.float().cpu().numpy()
    del buf, out
    y, _ = oracle.gemm(**oracle_args(w, t))
    assert tol_excess(got, y, 1e-3 if f32 else 2e-2) <= 0


def mapping_case(w: synth.Workload):
    """The integer-operand form of a workload at its real shape and storage:
    sparse +-1 rows against integers in [-4, 4] (bias in [-64, 64]) for bf16
    outputs, dense integers in [-2, 2] for fp32 outputs; linear workloads take
    the bias epilogue and the FFN the identity gate (g * u), whose results
    are exact small integers.  Returns (operands in storage layout, oracle
    keyword arguments, the call on the GPU)."""
    seed = (w.M * 31 + w.N * 7 + w.K) % 100003
    if w.out_dtype == "f32":
        A, B = synth.dense_int_operands(w.M, w.N, w.K, w.layout, seed)
        ops = dict(A=A, B=B)
        kw = dict(A=synth.bits(A), B=synth.bits(B), layout=w.layout, epilogue="none")
    elif w.form == "ffn":
        ops = synth.mapping_operands(w.M, w.N, w.K, "nt", seed, gated=True)
        ops = dict(A=ops["A"], B=ops["B"], B2=ops["B2"])
        kw = dict(A=synth.bits(ops["A"]), B=synth.bits(ops["B"]), B2=synth.bits(ops["B2"]),
                  layout="nt", epilogue="glu_identity")
    else:
        bias = w.form == "linear"
        o = synth.mapping_operands(w.M, w.N, w.K, w.layout, seed, with_bias=bias)
        ops = dict(A=o["A"], B=o["B"])
        kw = dict(A=synth.bits(o["A"]), B=synth.bits(o["B"]), layout=w.layout,
                  epilogue="bias" if bias else "none")
        if bias:
            ops["bias"] = o["bias"]
            kw["bias"] = synth.bits(o["bias"])
    return ops, kw


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_mapping_bitexact(dev, name):
    """Tile order, index mapping and K slicing bit for bit at each workload's
    real shape, storage and launch configuration (persistent grid, XCD remap,
    band order, K alternation, automatic split-K): integer operands whose
    fp32 sums are exact in any order, every output element compared with the
    oracle's bits, guard bands checked."""
    w = synth.WORKLOADS[name]
    say("workload mapping", name, binding.describe_config(w.form, w.M, w.N, w.K, w.layout))
    ops, kw = mapping_case(w)
    f32 = w.out_dtype == "f32"
    buf, out = guarded_out(w.M, w.N, f32, dev)
    g = {k: v.to(dev) for k, v in ops.items()}
    lay = w.layout
    if w.form == "ffn":
        call_ffn(g["A"], g["B"], g["B2"], w.M, w.N, w.K, "identity", out)
    else:
        # the bench's call: torch views of the stored operands, read in place
        A = g["A"].t() if lay[0] == "t" else g["A"]
        B = g["B"].t() if lay[1] == "t" else g["B"]
        if w.form == "linear":
            mm.linear(A, g["B"], g["bias"], "bias", out=out)
        else:
            mm.matmul(A, B, torch.float32 if f32 else torch.bfloat16, out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, w.M, w.N)
    got = out.cpu()
    del buf, out, g
    ref, ref_bits = oracle.gemm(**kw)
    if f32:
        bad = np.argwhere(got.numpy() != ref)
    else:
        bad = np.argwhere(to_bits(got) != ref_bits)
    assert bad.size == 0, f"{name}: {len(bad)} mismatches, first {bad[:5].tolist()}"


# shapes the heuristic gives 256 x 192 tiles (fewer passes of the grid than
# 256 x 256): one full pass, one with ragged last tile rows and columns, and
# three passes
NARROW_SHAPES = [(3072, 3072, 3072), (2900, 3000, 2048), (6144, 6144, 6144)]


@pytest.mark.parametrize("shape", NARROW_SHAPES)
def test_narrow_tiles_default_path(dev, shape):
    """The default configuration's 256 x 192 tiles: the index mapping bit for
    bit with integer operands (every output element, guard bands), and
    linear + bias + GELU on random operands within the bf16 tolerance."""
    M, N, K = shape
    cfg = binding.describe_config("linear", M, N, K)
    say("narrow tiles", shape, cfg)
    assert cfg.startswith("BM=256,BN=192") and cfg.endswith("KERNEL=gemm_nt_slab"), cfg
    ops = synth.mapping_operands(M, N, K, "nt", seed=M + N + K, with_bias=True)
    buf, out = guarded_out(M, N, False, dev)
    mm.linear(ops["A"].to(dev), ops["B"].to(dev), ops["bias"].to(dev), "bias", out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    got = to_bits(out)
    _, bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), "nt", "bias",
                          bias=synth.bits(ops["bias"]))
    bad = np.argwhere(got != bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    x = synth.randn_bf16((M, K), 1.0, 51)
    W = synth.randn_bf16((N, K), K ** -0.5, 52)
    b = synth.randn_bf16((N,), 1.0, 53)
    got = mm.linear(x.to(dev), W.to(dev), b.to(dev), "bias_gelu_tanh")
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(x), synth.bits(W), "nt", "bias_gelu_tanh", bias=synth.bits(b))
    assert tol_excess(got.float().cpu().numpy(), y, 2e-2) <= 0


# K not a multiple of 64 on the default path: the slab kernel's last
# super-step of every tile is a partial one (its copies fetch zeros past K).
# 256 x 192 tiles with a 56-k and an 8-k tail (the first with K alternation,
# so half the tiles start with the partial super-step), 256 x 256 tiles with
# an 8-k tail, and a mid-size shape that the heuristic gives 128 x 128 tiles.
RAGGED_SHAPES = [(3000, 3000, 3000), (2900, 3000, 1032), (4096, 4096, 4168), (1000, 1000, 3080)]


@pytest.mark.parametrize("shape", RAGGED_SHAPES)
def test_ragged_k_default_path(dev, shape):
    """Every output element bit for bit with integer operands (guard bands
    checked), then linear + bias + GELU on random operands within the bf16
    tolerance, and an fp32 matmul of dense integers bit for bit."""
    M, N, K = shape
    cfg = binding.describe_config("linear", M, N, K)
    say("ragged K", shape, cfg)
    if M * N >= 2000 * 2000:
        assert cfg.endswith("KERNEL=gemm_nt_slab"), cfg
    ops = synth.mapping_operands(M, N, K, "nt", seed=M + N + K, with_bias=True)
    buf, out = guarded_out(M, N, False, dev)
    mm.linear(ops["A"].to(dev), ops["B"].to(dev), ops["bias"].to(dev), "bias", out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    _, bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), "nt", "bias",
                          bias=synth.bits(ops["bias"]))
    bad = np.argwhere(to_bits(out) != bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    del buf, out
    x = synth.randn_bf16((M, K), 1.0, 61)
    W = synth.randn_bf16((N, K), K ** -0.5, 62)
    b = synth.randn_bf16((N,), 1.0, 63)
    got = mm.linear(x.to(dev), W.to(dev), b.to(dev), "bias_gelu_tanh")
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(x), synth.bits(W), "nt", "bias_gelu_tanh", bias=synth.bits(b))
    assert tol_excess(got.float().cpu().numpy(), y, 2e-2) <= 0
    A, B = synth.dense_int_operands(M, N, K, "nt", seed=7)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    call_matmul(A.to(dev), B.to(dev), M, N, K, "nt", True, out)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(synth.bits(A), synth.bits(B), "nt")
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_ragged_k_ffn_default_path(dev):
    """The FFN with K not a multiple of 64 on the default path: bit for bit
    with the identity gate and integer operands (guard bands checked), SwiGLU
    on random operands within the bf16 tolerance."""
    M, N, K = 2000, 3000, 1000
    cfg = binding.describe_config("ffn", M, N, K)
    say("ragged K ffn", (M, N, K), cfg)
    assert cfg.endswith("KERNEL=gemm_nt_slab"), cfg
    ops = synth.mapping_operands(M, N, K, "nt", seed=77, gated=True)
    buf, out = guarded_out(M, N, False, dev)
    call_ffn(ops["A"].to(dev), ops["B"].to(dev), ops["B2"].to(dev), M, N, K, "identity", out)
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    _, bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), "nt", "glu_identity",
                          B2=synth.bits(ops["B2"]))
    bad = np.argwhere(to_bits(out) != bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    del buf, out
    x = synth.randn_bf16((M, K), 1.0, 71)
    Wg = synth.randn_bf16((N, K), K ** -0.5, 72)
    Wu = synth.randn_bf16((N, K), K ** -0.5, 73)
    got = mm.ffn_swiglu(x.to(dev), Wg.to(dev), Wu.to(dev))
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(x), synth.bits(Wg), "nt", "swiglu", B2=synth.bits(Wu))
    assert tol_excess(got.float().cpu().numpy(), y, 2e-2) <= 0


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_ragged_k_transposed_storage(dev, layout):
    """K not a multiple of 64 with operands stored [K][N] and/or [K][M] on the
    default path (the transpose-read slab forms; their k-rows past K lie past
    the end of the matrix): bit for bit with integer operands, bf16 with a
    bias and fp32, guard bands checked."""
    M, N, K = 4000, 3000, 1032
    cfg = binding.describe_config("linear", M, N, K, layout)
    say("ragged K", layout, (M, N, K), cfg)
    assert cfg.endswith("KERNEL=gemm_nt_slab"), cfg
    ops = synth.mapping_operands(M, N, K, layout, seed=M + N + K + 1, with_bias=True)
    buf, out = guarded_out(M, N, False, dev)
    call_linear(ops["A"].to(dev), ops["B"].to(dev), ops["bias"].to(dev), M, N, K, layout, "bias", out)
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    _, bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), layout, "bias",
                          bias=synth.bits(ops["bias"]))
    bad = np.argwhere(to_bits(out) != bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    del buf, out
    A, B = synth.dense_int_operands(M, N, K, layout, seed=9)
    buf, out = guarded_out(M, N, True, dev)
    call_matmul(A.to(dev), B.to(dev), M, N, K, layout, True, out)
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    ref, _ = oracle.gemm(synth.bits(A), synth.bits(B), layout)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
def test_batched_ragged_k_slab(dev, layout):
    """Batched products with K not a multiple of 64 on the slab kernel (a
    small grid: several units per workgroup, K alternating): each entry's
    k-rows past K, for operands stored [K][N] or [K][M], end its record, so
    no entry reads its neighbour's values."""
    binding.set_config("BM=256,BN=256,WM=2,WN=2,G=2,XCD=0,KALT=1,GRID=3,PIPE=3")
    batch, M, N, K = 3, 264, 520, 1000
    say("batched ragged K", layout, (batch, M, N, K))
    As, Bs = [], []
    for b in range(batch):
        A, B = synth.dense_int_operands(M, N, K, layout, seed=300 + b)
        As.append(A)
        Bs.append(B)
    A_all = torch.stack(As).to(dev)
    B_all = torch.stack(Bs).to(dev)
    out = torch.full((batch, M, N), float("nan"), dtype=torch.float32, device=dev)
    call_matmul_batched(A_all, B_all, batch, M, N, K, As[0].numel(), Bs[0].numel(), M * N, layout, True,
                        out)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, _ = oracle.gemm(synth.bits(As[b]), synth.bits(Bs[b]), layout)
        np.testing.assert_array_equal(out[b].cpu().numpy(), ref)


# ------------------------------------------------------------ skinny products
# (M, N, K): at most 32 activation rows against at least 8 MiB of weights --
# ragged N and K (multiples of 8), slices of K that end mid-stage, one row,
# an M*N that is not a multiple of 4 (the reduction's scalar path); one and
# two blocks of 16 activation rows, full and partial
SKINNY_SHAPES = [(1, 4096, 1024), (7, 1000, 8200), (16, 8192, 1032), (9, 4104, 4096), (16, 2048, 2056),
                 (13, 3000, 4096), (2, 1032, 8192), (7, 1001, 8200), (17, 4104, 4096), (32, 2048, 2056),
                 (27, 1001, 8200), (32, 8192, 1032)]


@pytest.mark.parametrize("shape", SKINNY_SHAPES)
@pytest.mark.parametrize("ws", [False, True])
def test_skinny_mapping_bitexact(dev, shape, ws):
    """The skinny kernel, unsplit (no workspace) and with K cut into slices
    (a workspace): bf16 with a bias from integer operands, and fp32 from
    dense integers, against the oracle's bits; guard bands checked."""
    M, N, K = shape
    cfg = binding.describe_config("linear", M, N, K)
    say("skinny", shape, "ws" if ws else "no ws", cfg)
    assert cfg.endswith("KERNEL=gemm_skinny"), cfg
    nbytes = binding.workspace_size("linear", M, N, K) if ws else 0
    wsp = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=dev)
    lib = binding.load()
    ops = synth.mapping_operands(M, N, K, "nt", seed=M + 3 * N + K, with_bias=True)
    A, B, bias = ops["A"].to(dev), ops["B"].to(dev), ops["bias"].to(dev)
    buf, out = guarded_out(M, N, False, dev)
    st = lib.mm_linear_ws(A.data_ptr(), B.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K,
                          binding.LAYOUTS["nt"], binding.EPILOGUES["bias"], wsp.data_ptr() if ws else None,
                          nbytes, stream())
    binding.check(st, "mm_linear_ws")
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    _, bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), "nt", "bias", bias=synth.bits(ops["bias"]))
    np.testing.assert_array_equal(to_bits(out), bits)
    del buf, out
    Ad, Bd = synth.dense_int_operands(M, N, K, "nt", seed=M + N)
    buf, out = guarded_out(M, N, True, dev)
    st = lib.mm_matmul_ws(Ad.to(dev).data_ptr(), Bd.to(dev).data_ptr(), out.data_ptr(), M, N, K,
                          binding.LAYOUTS["nt"], 1, wsp.data_ptr() if ws else None, nbytes, stream())
    binding.check(st, "mm_matmul_ws")
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N)
    ref, _ = oracle.gemm(synth.bits(Ad), synth.bits(Bd), "nt")
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("shape", [(16, 8192, 8192), (5, 4096, 4104), (32, 4096, 8192), (29, 8192, 4096)])
@pytest.mark.parametrize("epi", ["bias_gelu_tanh", "gelu_tanh", "none"])
def test_skinny_random(dev, shape, epi):
    """Random operands through mm.linear (its automatic workspace: K in
    slices) within the bf16 tolerance; run to run identical."""
    M, N, K = shape
    say("skinny random", shape, epi)
    x = synth.randn_bf16((M, K), 1.0, 91)
    W = synth.randn_bf16((N, K), K ** -0.5, 92)
    b = synth.randn_bf16((N,), 1.0, 93)
    bd = b.to(dev) if "bias" in epi else None
    o1 = mm.linear(x.to(dev), W.to(dev), bd, epi)
    o2 = mm.linear(x.to(dev), W.to(dev), bd, epi)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    y, _ = oracle.gemm(synth.bits(x), synth.bits(W), "nt", epi, bias=synth.bits(b) if bd is not None else None)
    assert tol_excess(o1.float().cpu().numpy(), y, 2e-2) <= 0


# ------------------------------------------------------------ non-finite inputs
def nonfinite_case(M, N, K, layout, seed):
    """op(A) [M,K], op(B) [K,N] (bf16, N(0,1)-like) with +-inf and NaN entries
    spread over several tiles and k positions: an inf above a zero of op(B)
    (inf * 0), a NaN row, a -inf in op(B), and +inf / -inf in one row of
    op(A).  Returns storage-layout tensors and the per-output IEEE class (0
    finite, 1 +inf, -1 -inf, 2 NaN), which no summation order changes."""
    a = synth.randn_bf16((M, K), 1.0, seed).float()
    b = synth.randn_bf16((K, N), K ** -0.5, seed + 1).float()
    inf, nan = float("inf"), float("nan")
    for (i, k) in [(1, 2), (M - 1, K - 1), (M // 2, K // 3)]:
        a[i, k] = inf
    b[2, N - 1] = 0.0
    a[min(2, M - 1), K // 2] = nan
    b[K - 5, min(6, N - 1)] = -inf
    b[K // 4, N // 2] = inf
    a[min(3, M - 1), 7] = inf
    a[min(3, M - 1), K - 8] = -inf
    # only k positions holding a non-finite entry can make an output
    # non-finite (the finite terms are small: no finite sum overflows)
    ks = torch.nonzero(~torch.isfinite(a).all(0) | ~torch.isfinite(b).all(1)).flatten()
    t = a.double()[:, ks, None] * b.double()[None, ks, :]
    pos, neg = torch.isposinf(t).any(1), torch.isneginf(t).any(1)
    isnan = torch.isnan(t).any(1) | (pos & neg)
    cls = torch.where(isnan, 2, torch.where(pos, 1, torch.where(neg, -1, 0))).numpy()
    a, b = a.to(torch.bfloat16), b.to(torch.bfloat16)
    A = a.t().contiguous() if layout in ("tn", "tt") else a
    B = b.t().contiguous() if layout in ("nt", "tt") else b
    return A, B, cls


def value_class(y):
    y = np.asarray(y, np.float64)
    return np.where(np.isnan(y), 2, np.where(np.isposinf(y), 1, np.where(np.isneginf(y), -1, 0)))


# (configuration, M, N, K, layout): the slab kernel (ragged K, [K][N] weights,
# 256 x 192 tiles), the 32-k pipeline, the all-of-K-in-LDS small kernel and
# the basic kernel
NONFINITE_CASES = [
    (CONFIGS[1], 520, 395, 1032, "nt"),
    (CONFIGS[0], 520, 392, 1024, "nn"),
    ("BM=256,BN=192,WM=2,WN=2,G=4,XCD=1,KALT=1,PIPE=3", 520, 395, 1024, "nt"),
    (CONFIGS[3], 520, 395, 1024, "nt"),
    ("BM=64,BN=64,WM=2,WN=2,G=3,XCD=0,KALT=0,GRID=3", 300, 264, 200, "nt"),
    ("BM=64,BN=64,WM=2,WN=2,G=3,XCD=0,KALT=0,PIPE=0", 304, 264, 200, "tn"),
]


@pytest.mark.parametrize("case", range(len(NONFINITE_CASES)))
@pytest.mark.parametrize("epi", ["none", "bias_gelu_tanh"])
def test_nonfinite_inputs(dev, case, epi):
    """Inf and NaN in the operands: every output has the oracle's class
    (finite, +inf, -inf, NaN; GELU(-inf) is NaN), and the finite outputs are
    within the bf16 tolerance."""
    cfg, M, N, K, layout = NONFINITE_CASES[case]
    binding.set_config(cfg)
    say("non-finite", cfg, (M, N, K), layout, epi)
    A, B, cls = nonfinite_case(M, N, K, layout, 31 + case)
    bias = synth.randn_bf16((N,), 1.0, 39)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    call_linear(A.to(dev), B.to(dev), bias.to(dev), M, N, K, layout, epi, out)
    torch.cuda.synchronize()
    y, bits = oracle.gemm(synth.bits(A), synth.bits(B), layout, epi, bias=synth.bits(bias))
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    got = out.float().cpu().numpy()
    if epi == "none":
        np.testing.assert_array_equal(value_class(ref), cls)  # the oracle agrees with IEEE
    np.testing.assert_array_equal(value_class(got), value_class(ref))
    fin = value_class(ref) == 0
    excess = np.abs(got[fin].astype(np.float64) - y[fin]) - 2e-2 * (np.abs(y[fin]) + 1.0)
    assert excess.max() <= 0


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("epi", ["none", "bias_gelu_tanh"])
def test_nonfinite_inputs_skinny(dev, ws, epi):
    """The same classes through the skinny kernel: 13 rows (one block of 16)
    and 29 (two), unsplit and with K in slices (fp32 partial sums added by
    the reduction: +inf in one slice and -inf in another give NaN)."""
    binding.set_config(None)
    for (M, N, K) in [(13, 4104, 2056), (29, 2056, 4104)]:
        say("non-finite skinny", (M, N, K), epi, "ws" if ws else "no ws")
        assert binding.describe_config("linear", M, N, K).endswith("KERNEL=gemm_skinny")
        A, B, cls = nonfinite_case(M, N, K, "nt", 47 + M)
        bias = synth.randn_bf16((N,), 1.0, 49)
        nbytes = binding.workspace_size("linear", M, N, K)
        assert nbytes > 0 or not ws, "shape no longer split"
        wsp = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if ws else None
        out = mm.linear(A.to(dev), B.to(dev), bias.to(dev), epi, workspace=wsp)
        torch.cuda.synchronize()
        y, bits = oracle.gemm(synth.bits(A), synth.bits(B), "nt", epi, bias=synth.bits(bias))
        ref = (bits.astype(np.uint32) << 16).view(np.float32)
        got = out.float().cpu().numpy()
        if epi == "none":
            np.testing.assert_array_equal(value_class(ref), cls)
        np.testing.assert_array_equal(value_class(got), value_class(ref))
        fin = value_class(ref) == 0
        excess = np.abs(got[fin].astype(np.float64) - y[fin]) - 2e-2 * (np.abs(y[fin]) + 1.0)
        assert excess.max() <= 0


def test_nonfinite_inputs_split_and_ffn(dev):
    """The same classes through split-K (partial tiles added by the
    reduction) and through the FFN's SwiGLU (SiLU(-inf) u is NaN)."""
    M, N, K = 520, 392, 8192
    A, B, cls = nonfinite_case(M, N, K, "nt", 41)
    assert binding.workspace_size("matmul", M, N, K, "nt") > 0, "shape no longer split"
    ws = torch.empty(binding.workspace_size("matmul", M, N, K, "nt"), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    say("non-finite split-K", (M, N, K))
    mm.matmul(A.to(dev), B.to(dev).t(), torch.float32, out=out, workspace=ws)
    torch.cuda.synchronize()
    y, _ = oracle.gemm(synth.bits(A), synth.bits(B), "nt")
    np.testing.assert_array_equal(value_class(y), cls)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(value_class(got), cls)
    fin = cls == 0
    assert tol_excess(got[fin], y[fin], 1e-3) <= 0
    M, N, K = 300, 264, 1032
    x, Wg, _ = nonfinite_case(M, N, K, "nt", 43)
    Wu = synth.randn_bf16((N, K), K ** -0.5, 45)
    Wu[5, :] = 0.0  # SiLU(+-inf) * 0 = NaN as well
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("non-finite ffn", (M, N, K))
    mm.ffn_swiglu(x.to(dev), Wg.to(dev), Wu.to(dev), out=out)
    torch.cuda.synchronize()
    y, bits = oracle.gemm(synth.bits(x), synth.bits(Wg), "nt", "swiglu", B2=synth.bits(Wu))
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    got = out.float().cpu().numpy()
    np.testing.assert_array_equal(value_class(got), value_class(ref))
    fin = value_class(ref) == 0
    assert tol_excess(got[fin], y[fin], 2e-2) <= 0


# ------------------------------------------------------------ edge cases
def test_empty_and_tiny(dev):
    say("empty and tiny")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((16, 64), dtype=torch.bfloat16, device=dev)
    assert mm.linear(x, W).shape == (0, 16)
    assert mm.matmul(torch.zeros((5, 8), dtype=torch.bfloat16, device=dev),
                     torch.zeros((8, 0), dtype=torch.bfloat16, device=dev)).shape == (5, 0)
    a = synth.randn_bf16((1, 8), 1.0, 9)
    b = synth.randn_bf16((8, 1), 1.0, 10)
    got = mm.matmul(a.to(dev), b.t().contiguous().to(dev).t(), torch.float32)
    y, _ = oracle.gemm(synth.bits(a), synth.bits(b), "nn")
    assert tol_excess(got.cpu().numpy(), y, 1e-3) <= 0


def test_empty_sum_k0(dev):
    """K = 0: every accumulator is the empty sum 0, so each form's output is
    its epilogue applied to 0 + bias, which the oracle's loop with no k terms
    gives too: bias exactly, GELU(bias) within the GELU tolerance, zeros for
    the plain and FFN products.  Operands are empty (null pointers through
    the C ABI); outputs start as 0xFF bytes, so every element must be
    written."""
    M, N = 37, 300
    say("K = 0", (M, N))
    bias = synth.randn_bf16((N,), 1.0, 91)
    bias_d = bias.to(dev)
    Ah, Bh = np.zeros((M, 0), np.uint16), np.zeros((N, 0), np.uint16)
    lib = binding.load()
    for f32 in (False, True):
        out = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device=dev)
        out.view(torch.uint8).fill_(0xFF)
        binding.check(lib.mm_matmul(None, None, out.data_ptr(), M, N, 0, binding.LAYOUTS["nn"],
                                    1 if f32 else 0, stream()), "mm_matmul")
        assert torch.all(out == 0)
    for epi in ("none", "bias", "gelu_tanh", "bias_gelu_tanh"):
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        out.view(torch.uint8).fill_(0xFF)
        b = bias_d if "bias" in epi else None
        binding.check(lib.mm_linear(None, None, b.data_ptr() if b is not None else None, out.data_ptr(),
                                    M, N, 0, binding.LAYOUTS["nt"], binding.EPILOGUES[epi], stream()),
                      "mm_linear")
        y, bits = oracle.gemm(Ah, Bh, "nt", epi, bias=synth.bits(bias) if b is not None else None)
        if "gelu" in epi:
            assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0, epi
        else:
            np.testing.assert_array_equal(to_bits(out), bits, err_msg=epi)
    # the two-output form: the pre-activation is the bias itself
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    pre = torch.empty_like(out)
    call_linear_preact(torch.empty((M, 0), dtype=torch.bfloat16, device=dev),
                       torch.empty((N, 0), dtype=torch.bfloat16, device=dev), bias_d, M, N, 0, "nt",
                       "bias_gelu_tanh", out, pre)
    y, _ = oracle.gemm(Ah, Bh, "nt", "bias_gelu_tanh", bias=synth.bits(bias))
    np.testing.assert_array_equal(to_bits(pre), np.broadcast_to(synth.bits(bias), (M, N)))
    assert tol_excess(out.float().cpu().numpy(), y, 2e-2) <= 0
    # FFN forms: act(0) * 0 = 0
    for act in ("silu", "identity"):
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        out.view(torch.uint8).fill_(0xFF)
        binding.check(lib.mm_ffn_glu(None, None, None, out.data_ptr(), M, N, 0, binding.GLU_ACTS[act],
                                     stream()), "mm_ffn_glu")
        assert torch.all(out == 0), act
    # batched with a shared bias, and through the torch-facing wrappers
    x3 = torch.empty((3, M, 0), dtype=torch.bfloat16, device=dev)
    got = mm.linear_batched(x3, torch.empty((N, 0), dtype=torch.bfloat16, device=dev), bias_d, "bias")
    for e in range(3):
        np.testing.assert_array_equal(to_bits(got[e]), np.broadcast_to(synth.bits(bias), (M, N)))
    got = mm.matmul(torch.empty((M, 0), dtype=torch.bfloat16, device=dev),
                    torch.empty((0, N), dtype=torch.bfloat16, device=dev), torch.float32)
    torch.cuda.synchronize()
    assert got.shape == (M, N) and torch.all(got == 0)


def test_unaligned_output_rows_and_pointer(dev):
    """fp32 rows of 3001 elements (12004 bytes, not 16-byte multiples) and a
    bf16 output that starts 2 bytes past a 16-byte boundary."""
    M, N, K = 70, 3001, 136
    say("unaligned output", (M, N, K))
    A, B = synth.dense_int_operands(M, N, K, "nt", seed=77)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    call_matmul(A.to(dev), B.to(dev), M, N, K, "nt", True, out)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(synth.bits(A), synth.bits(B), "nt")
    np.testing.assert_array_equal(out.cpu().numpy(), ref)
    M, N = 40, 64
    ops = synth.mapping_operands(M, N, K, "nt", seed=78, with_bias=True)
    buf = torch.zeros(M * N + 8, dtype=torch.bfloat16, device=dev)
    out = buf[1:1 + M * N].view(M, N)
    call_linear(ops["A"].to(dev), ops["B"].to(dev), ops["bias"].to(dev), M, N, K, "nt", "bias", out)
    torch.cuda.synchronize()
    _, ref_bits = oracle.gemm(synth.bits(ops["A"]), synth.bits(ops["B"]), "nt", "bias",
                              bias=synth.bits(ops["bias"]))
    np.testing.assert_array_equal(to_bits(out), ref_bits)
    assert buf[0].item() == 0 and torch.all(buf[1 + M * N:] == 0)


@pytest.mark.parametrize("cfg", CONFIGS[:2])
@pytest.mark.parametrize("K", [200, 192])
def test_guard_bands_untouched(dev, cfg, K):
    binding.set_config(cfg)
    M, N = 259, 261
    say("guard bands", cfg, K)
    guard = 2048  # elements = 4 KiB of fp32
    A, B = synth.dense_int_operands(M, N, K, "nt", seed=5)
    buf = torch.full((M * N + 2 * guard,), 12345.0, dtype=torch.float32, device=dev)
    out = buf[guard:guard + M * N].view(M, N)
    call_matmul(A.to(dev), B.to(dev), M, N, K, "nt", True, out)
    torch.cuda.synchronize()
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + M * N:] == 12345.0)


def test_repeatable_bitwise(dev):
    w = synth.WORKLOADS["linear_bias_gelu_4096"]
    say("repeatable", w.name)
    t = w.make()
    o1 = run_workload(w, t, dev).clone()
    o2 = run_workload(w, t, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_no_device_allocation_per_call(dev):
    w = synth.WORKLOADS["linear_bias_gelu_4096"]
    t = {k: v.to(dev) for k, v in w.make().items()}
    out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    mm.linear(t["x"], t["W"], t["bias"], w.epilogue, out=out)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(3):
        mm.linear(t["x"], t["W"], t["bias"], w.epilogue, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before


def test_torch_views_map_to_layouts(dev):
    """A .t() view of a contiguous tensor is read in place as the matching layout."""
    M, N, K = 136, 72, 96
    say("views")
    a = synth.randint_bf16((M, K), -3, 3, 1)
    b = synth.randint_bf16((K, N), -3, 3, 2)
    want = (a.float() @ b.float()).numpy()
    for A in (a.to(dev), a.t().contiguous().to(dev).t()):
        for B in (b.to(dev), b.t().contiguous().to(dev).t()):
            got = mm.matmul(A, B, torch.float32)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got.cpu().numpy(), want)
    with pytest.raises(ValueError):
        mm.matmul(a.to(dev)[:, ::2], b.to(dev)[::2])


def test_int64_operand_offsets(dev):
    """A has 32769 x 65536 = 2^31 + 65536 elements: its last rows sit past the
    32-bit element range.  Checks the last 64 output rows."""
    M, N, K = 32769, 128, 65536
    say("int64 offsets", (M, N, K))
    free, _total = torch.cuda.mem_get_info()
    if free < 12 * 2 ** 30:
        pytest.skip("needs ~12 GiB of free device memory")
    g = torch.Generator(device=dev).manual_seed(601)
    A = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    B = synth.randn_bf16((N, K), K ** -0.5, 602)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    call_matmul(A, B.to(dev), M, N, K, "nt", True, out)
    torch.cuda.synchronize()
    rows = A[M - 64:].cpu()
    del A
    y, _ = oracle.gemm(synth.bits(rows), synth.bits(B), "nt")
    assert tol_excess(out[M - 64:].cpu().numpy(), y, 1e-3) <= 0


@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_int64_transposed_storage(dev, layout):
    """The operand stored [K][M] (tn) or [K][N] (nn) has 65536 x 32776 =
    2^31 + 524288 elements: the k-row offsets of the transpose-read kernels pass
    2^32 bytes, and the buffer range is capped.  Checks the 64 outputs nearest
    the operand's end (last rows for tn, last columns for nn)."""
    K, big, small = 65536, 32776, 128
    M, N = (big, small) if layout == "tn" else (small, big)
    say("int64 transposed storage", layout, (M, N, K))
    free, _total = torch.cuda.mem_get_info()
    if free < 14 * 2 ** 30:
        pytest.skip("needs ~14 GiB of free device memory")
    g = torch.Generator(device=dev).manual_seed(603)
    # N(0, 1) activations, N(0, 1/K) weights: outputs of order 1, as in the workloads
    sigma = 1.0 if layout == "tn" else K ** -0.5
    Big = torch.randn((K, big), generator=g, device=dev, dtype=torch.float32).mul_(sigma).to(torch.bfloat16)
    other = synth.randn_bf16((K, small), K ** -0.5, 604)
    A, B = (Big, other.to(dev)) if layout == "tn" else (other.to(dev), Big)
    if layout == "nn":  # A [M][K]
        A = synth.randn_bf16((M, K), 1.0, 605).to(dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    # the 256 x 256 slab kernel (the heuristic would take 128 x 128 tiles here)
    binding.set_config("BM=256,BN=256,WM=2,WN=2,PIPE=3")
    assert binding.describe_config("matmul", M, N, K, layout).endswith("KERNEL=gemm_nt_slab")
    call_matmul(A, B, M, N, K, layout, True, out)
    torch.cuda.synchronize()
    tail = Big[:, big - 64:].contiguous().cpu()
    del Big, A, B
    if layout == "tn":
        y, _ = oracle.gemm(synth.bits(tail), synth.bits(other), "tn")
        got = out[M - 64:].cpu().numpy()
    else:
        Ah = synth.randn_bf16((M, K), 1.0, 605)
        y, _ = oracle.gemm(synth.bits(Ah), synth.bits(tail), "nn")
        got = out[:, N - 64:].cpu().numpy()
    assert tol_excess(got, y, 1e-3) <= 0


def test_bias_staged_workload_mapping(dev):
    """The bias-staging instance at the 8192^3 linear workload's real shape and
    launch (BSTAGE=1 on the heuristic's tile order): integer operands, bias
    epilogue, every output bit equal to the oracle's."""
    w = synth.WORKLOADS["linear_bias_gelu_8192"]
    cfg = binding.describe_config(w.form, w.M, w.N, w.K, w.layout).rsplit(",KERNEL=", 1)[0] + ",BSTAGE=1"
    binding.set_config(cfg)
    say("bias staged mapping", cfg)
    ops, kw = mapping_case(w)
    buf, out = guarded_out(w.M, w.N, False, dev)
    g = {k: v.to(dev) for k, v in ops.items()}
    mm.linear(g["A"], g["B"], g["bias"], "bias", out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, w.M, w.N)
    got = out.cpu()
    del buf, out, g
    _, ref_bits = oracle.gemm(**kw)
    bad = np.argwhere(to_bits(got) != ref_bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


@pytest.mark.parametrize("name", ["linear_bias_gelu_8192", "linear_bias_gelu_4096"])
def test_pingpong_workload_mapping(dev, name):
    """The two-group ping-pong kernel (PIPE=5) at the linear workloads' real
    shapes: integer operands, bias epilogue, every output bit equal to the
    oracle's, guard bands intact."""
    w = synth.WORKLOADS[name]
    binding.set_config("BM=256,BN=128,WM=2,WN=4,G=4,XCD=1,KALT=0,PIPE=5")
    assert binding.describe_config(w.form, w.M, w.N, w.K, w.layout).endswith("KERNEL=gemm_pp")
    say("ping-pong mapping", name)
    ops, kw = mapping_case(w)
    buf, out = guarded_out(w.M, w.N, False, dev)
    g = {k: v.to(dev) for k, v in ops.items()}
    mm.linear(g["A"], g["B"], g["bias"], "bias", out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, w.M, w.N)
    got = out.cpu()
    del buf, out, g
    _, ref_bits = oracle.gemm(**kw)
    bad = np.argwhere(to_bits(got) != ref_bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def test_splitk_tile_width_choice(dev):
    """The automatic split takes 256 x 192 tiles when they occupy more of the
    grid: the long-K workload's 128 such tiles in 2 chunks fill all 256 CUs
    (256 x 256 tiles: 96 in 2 chunks, 192 workgroups); a forced configuration
    and operands not stored K-contiguous keep 256 x 256."""
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the choice is stated for a 256-CU GPU")
    assert ",SPLIT=2x192," in binding.describe_config("matmul", 2047, 3001, 65536)
    assert ",SPLIT=2x192," in binding.describe_config("matmul", 2047, 3001, 65544)  # ragged K
    assert ",SPLIT=2x256," in binding.describe_config("matmul", 2047, 3001, 65536, "nn")
    binding.set_config("BM=256,BN=256,WM=2,WN=2,G=4,XCD=1,KALT=2,PIPE=3")
    try:
        assert ",SPLIT=2x256," in binding.describe_config("matmul", 2047, 3001, 65536)
    finally:
        binding.set_config(None)
    assert "SPLIT" not in binding.describe_config("matmul", 8192, 8192, 8192)
