"""mm_matmul_noalloc: the split-K product with the library's static scratch
instead of a caller's workspace, checked through the C ABI against
mm_matmul_ws (the same kernels with a workspace) and the oracle, on calls in
a row whose second input is smaller than the first."""

import numpy as np
import pytest
import torch

import oracle
from dense_bf16_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda:0")


def say(*a):
    print("case:", *a, flush=True)


def stream():
    return torch.cuda.current_stream().cuda_stream


def noalloc(A, B, M, N, K, layout, out_f32, out):
    st = binding.load().mm_matmul_noalloc(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                                         binding.LAYOUTS[layout], 1 if out_f32 else 0, stream())
    binding.check(st, "mm_matmul_noalloc")


def with_ws(A, B, M, N, K, layout, out_f32, out):
    nbytes = binding.workspace_size("matmul", M, N, K, layout)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=out.device)
    st = binding.load().mm_matmul_ws(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                                    binding.LAYOUTS[layout], 1 if out_f32 else 0,
                                    ws.data_ptr() if nbytes else None, nbytes, stream())
    binding.check(st, "mm_matmul_ws")
    torch.cuda.synchronize()
    return nbytes


# (M, N, K, layout): two calls in a row, the second smaller, both split by the
# automatic rule (32 tiles of 256 x 128 in 8 chunks: 256 slots, the whole
# 64 MiB of scratch; then 12 tiles in 10 chunks: 120 slots); then a stored-[K][N] product
# (256 x 256 tiles), a shape that runs unsplit, one whose K is not a
# multiple of 64 (never split: the slab kernel's ragged instance), a skinny
# product (16 rows: its fp32 partial outputs of 4 slices of K), and a skinny
# product whose one slice of partial outputs (67 MB) would not fit the
# scratch: it runs unsplit
SEQUENCE = [(1000, 900, 16384, "nt"), (520, 395, 8192, "nt"), (304, 264, 8192, "nn"),
            (520, 392, 512, "nt"), (2900, 3000, 1032, "nt"), (16, 4096, 8192, "nt"), (32, 524296, 256, "nt")]
UNSPLIT = {(520, 392, 512), (2900, 3000, 1032), (32, 524296, 256)}


@pytest.mark.parametrize("out_f32", [True, False])
def test_noalloc_matches_workspace_entry_point(dev, out_f32):
    for (M, N, K, layout) in SEQUENCE:
        say("noalloc", (M, N, K), layout, "f32" if out_f32 else "bf16")
        A, B = synth.dense_int_operands(M, N, K, layout, seed=M + 2 * N + K)
        Ad, Bd = A.to(dev), B.to(dev)
        dt = torch.float32 if out_f32 else torch.bfloat16
        got = torch.full((M, N), float("nan"), dtype=dt, device=dev)
        want = torch.full((M, N), float("nan"), dtype=dt, device=dev)
        noalloc(Ad, Bd, M, N, K, layout, out_f32, got)
        torch.cuda.synchronize()
        nbytes = with_ws(Ad, Bd, M, N, K, layout, out_f32, want)
        if (M, N, K) not in UNSPLIT:
            assert nbytes > 0, "this shape should take the split-K path"
        # same kernels, same partial sums, same order: identical bits
        assert torch.equal(got.view(torch.int32 if out_f32 else torch.int16),
                           want.view(torch.int32 if out_f32 else torch.int16))
        ref, bits = oracle.gemm(synth.bits(A), synth.bits(B), layout)
        if out_f32:
            np.testing.assert_array_equal(got.cpu().numpy(), ref)
        else:
            np.testing.assert_array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), bits)


def test_noalloc_random_data_and_no_allocation(dev):
    """N(0, 1) operands: bit-identical to the workspace call, within the fp32
    tolerance of the oracle; and the call leaves torch's allocator untouched."""
    M, N, K = 700, 900, 16384
    say("noalloc random", (M, N, K))
    x = synth.randn_bf16((M, K), 1.0, 71).to(dev)
    W = synth.randn_bf16((N, K), 2.0 ** -7, 72).to(dev)
    got = torch.empty((M, N), dtype=torch.float32, device=dev)
    want = torch.empty((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    noalloc(x, W, M, N, K, "nt", True, got)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    with_ws(x, W, M, N, K, "nt", True, want)
    assert torch.equal(got, want)
    y, _ = oracle.gemm(synth.bits(x.cpu()), synth.bits(W.cpu()), "nt")
    g = got.cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(g - y) - 1e-3 * (np.abs(y) + 1.0))) <= 0


def test_noalloc_rejects_what_the_scratch_cannot_hold(dev):
    """A forced stream-K split of 140 tiles in 4 chunks needs two slots for each
    of 187 workgroups (93.5 MiB), more than the 64 MiB scratch: refused with
    MM_ERR_UNSUPPORTED before any launch, the output untouched."""
    M, N, K = 2560, 3584, 2048
    binding.set_config("BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=2,SK=4")
    try:
        assert binding.workspace_size("matmul", M, N, K) > 64 << 20
        A = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
        B = torch.zeros((N, K), dtype=torch.bfloat16, device=dev)
        out = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
        with pytest.raises(binding.MMError) as e:
            noalloc(A, B, M, N, K, "nt", True, out)
        assert e.value.status == binding.MM_ERR_UNSUPPORTED
        assert "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    finally:
        binding.set_config(None)
