"""HIP graph capture of the library's launches.

Every entry point only enqueues kernels on the caller's stream (and allocates
nothing), so a sequence of calls can be captured into a HIP graph once and
replayed, the way a serving loop would issue them.  Each replay must equal
the eager calls bit for bit.  Replays are separated by eager work of the
program's own (the outputs are overwritten, other kernels run, the host
synchronizes), and every replay is checked, not just the first.  The cases
cover the slab kernel with a fused epilogue, the horizontally fused FFN, and
split-K with its two launches, through a caller's workspace and through the
library's static scratch, a split linear form whose reduction applies
the epilogue, a K that is not a multiple of 64 (the slab kernel's
ragged instance), and a skinny product (16 rows, K in slices, with its
reduction).
"""

import pytest
import torch

import dense_bf16_gemm_amd as mm
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


def noalloc(A, B, M, N, K, out):
    lib = binding.load()
    st = lib.mm_matmul_noalloc(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, binding.LAYOUTS["nt"],
                               1, torch.cuda.current_stream().cuda_stream)
    binding.check(st, "mm_matmul_noalloc")


def test_graph_replays_equal_eager_calls(dev):
    say("graph capture")
    # linear + bias + GELU on the slab kernel (interior and edge tiles)
    M, N, K = 1000, 1200, 1024
    x = synth.randn_bf16((M, K), 1.0, 801).to(dev)
    W = synth.randn_bf16((N, K), K ** -0.5, 802).to(dev)
    bias = synth.randn_bf16((N,), 1.0, 803).to(dev)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # FFN gate/up
    Mf, Nf, Kf = 512, 768, 512
    xf = synth.randn_bf16((Mf, Kf), 1.0, 804).to(dev)
    Wg = synth.randn_bf16((Nf, Kf), Kf ** -0.5, 805).to(dev)
    Wu = synth.randn_bf16((Nf, Kf), Kf ** -0.5, 806).to(dev)
    y2 = torch.empty((Mf, Nf), dtype=torch.bfloat16, device=dev)
    # a long-K product that the workspace splits (partial tiles, then their sum)
    Ms, Ns, Ks = 512, 520, 8192
    assert binding.workspace_size("matmul", Ms, Ns, Ks, "nt") > 0, "shape no longer split"
    As = synth.randn_bf16((Ms, Ks), 1.0, 807).to(dev)
    Bs = synth.randn_bf16((Ns, Ks), Ks ** -0.5, 808).to(dev)
    ws = torch.empty(binding.workspace_size("matmul", Ms, Ns, Ks, "nt"), dtype=torch.uint8, device=dev)
    y3 = torch.empty((Ms, Ns), dtype=torch.float32, device=dev)
    y4 = torch.empty((Ms, Ns), dtype=torch.float32, device=dev)
    # the same split with the linear form's epilogue, applied by the reduction
    bias_s = synth.randn_bf16((Ns,), 1.0, 809).to(dev)
    y5 = torch.empty((Ms, Ns), dtype=torch.bfloat16, device=dev)
    # K = 1032: every tile's last super-step is a partial one
    Mr, Nr, Kr = 2900, 3000, 1032
    assert binding.describe_config("linear", Mr, Nr, Kr).endswith("KERNEL=gemm_nt_slab")
    xr = synth.randn_bf16((Mr, Kr), 1.0, 810).to(dev)
    Wr = synth.randn_bf16((Nr, Kr), Kr ** -0.5, 811).to(dev)
    br = synth.randn_bf16((Nr,), 1.0, 812).to(dev)
    y6 = torch.empty((Mr, Nr), dtype=torch.bfloat16, device=dev)
    Mk, Nk, Kk = 16, 4096, 8192
    assert binding.describe_config("linear", Mk, Nk, Kk).endswith("KERNEL=gemm_skinny")
    xk = synth.randn_bf16((Mk, Kk), 1.0, 813).to(dev)
    Wk = synth.randn_bf16((Nk, Kk), Kk ** -0.5, 814).to(dev)
    wsk = torch.empty(max(binding.workspace_size("linear", Mk, Nk, Kk), 1), dtype=torch.uint8, device=dev)
    y7 = torch.empty((Mk, Nk), dtype=torch.bfloat16, device=dev)
    outs = (y1, y2, y3, y4, y5, y6, y7)

    def calls():
        mm.linear(x, W, bias, "bias_gelu_tanh", out=y1)
        mm.ffn_swiglu(xf, Wg, Wu, out=y2)
        mm.matmul(As, Bs.t(), torch.float32, out=y3, workspace=ws)
        noalloc(As, Bs, Ms, Ns, Ks, y4)
        mm.linear(As, Bs, bias_s, "bias_gelu_tanh", out=y5, workspace=ws)
        mm.linear(xr, Wr, br, "bias_gelu_tanh", out=y6)
        mm.linear(xk, Wk, None, "gelu_tanh", out=y7, workspace=wsk)

    calls()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert torch.equal(ref[2], ref[3]), "static scratch and caller workspace differ"

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    junk = torch.randn((2048, 2048), device=dev)
    for r in range(4):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5)
        junk = junk @ junk.t() * 1e-3  # other eager kernels between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            same = torch.equal(o.view(torch.uint8), e.view(torch.uint8))
            assert same, f"replay {r}: output {i} differs from the eager call"
    del g
