"""PyTorch-facing wrappers of the C ABI: shape/stride checks, output
allocation and the current stream.  No arithmetic happens here.

Transposed operands are passed as views (``t.t()`` of a contiguous tensor);
the layout letters tell the kernel how to read them in place.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding


def _letter(t: torch.Tensor, name: str) -> str:
    """'n' if the logical 2-D operand is stored as-is, 't' if it is the
    transpose of a contiguous matrix.  Anything else is refused (no copies)."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    as_is, transposed = t.is_contiguous(), t.t().is_contiguous()
    if as_is and transposed:  # a dimension of size 1: both describe the memory
        return "n" if t.shape[1] >= t.shape[0] else "t"
    if as_is:
        return "n"
    if transposed:
        return "t"
    raise ValueError(f"{name} must be contiguous or the transpose of a contiguous tensor")


def _check(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# One split-K workspace per (device, stream), grown on demand.  Calls on one
# stream share it (a call reads only slots it has written itself, in stream
# order); each stream has its own, so calls in flight on different streams do
# not race on it.  The tensor is allocated while its stream is current, so the
# caching allocator reuses its memory, after it is replaced, only in that
# stream's order.
_workspaces: dict = {}


def _workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, torch.cuda.current_stream(index).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def release_workspaces(device=None) -> None:
    """Drops the cached split-K workspaces (all devices, or one), so their
    memory returns to torch's caching allocator.  Call it after the work of
    every stream that used them has been synchronized; later split-K calls
    allocate a new one on demand."""
    if device is None:
        _workspaces.clear()
        return
    index = torch.device(device).index
    if index is None:
        index = torch.cuda.current_device()
    for key in [k for k in _workspaces if k[0] == index]:
        del _workspaces[key]


def _resolve_ws(workspace, form: str, M: int, N: int, K: int, layout: str, device):
    """(pointer, bytes) of the split-K workspace: "auto" uses the current
    stream's cached one, sized by mm_workspace_size; None disables split-K; a
    uint8 tensor is used as given."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 tensor')
        nbytes = binding.workspace_size(form, M, N, K, layout) if M and N and K else 0
        if nbytes == 0:
            return None, 0
        workspace = _workspace(nbytes, device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the operands' device")
    return workspace.data_ptr(), workspace.numel()


def matmul(A: torch.Tensor, B: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
           out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """MatmulOp form: out = A @ B with A [M,K] and B [K,N] (either may be a
    transposed view), fp32 accumulation, bf16 or fp32 output.  `workspace`
    enables split-K for shapes with too few output tiles (see
    mm_workspace_size): "auto", None (off) or a uint8 tensor."""
    _check(A, "A")
    _check(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    layout = _letter(A, "A") + _letter(B, "B")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of out_dtype")
    lib = binding.load()
    wp, wb = _resolve_ws(workspace, "matmul", M, N, K, layout, A.device)
    st = lib.mm_matmul_ws(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                          binding.LAYOUTS[layout],
                          binding.OUT_DTYPES["f32" if out_dtype == torch.float32 else "bf16"], wp, wb,
                          _stream())
    binding.check(st, "mm_matmul_ws")
    return out


def linear(x: torch.Tensor, W: torch.Tensor, bias: Optional[torch.Tensor] = None,
           epilogue: str = "none", out: Optional[torch.Tensor] = None,
           workspace="auto") -> torch.Tensor:
    """LinearOp form: out = epi(x @ W.T + bias) with x [M,K], W [N,K], bias [N],
    epilogue one of none | bias | gelu_tanh | bias_gelu_tanh; bf16 output.
    `workspace` as for matmul (a split product's reduction applies the
    epilogue to the summed value)."""
    _check(x, "x")
    _check(W, "W")
    M, K = x.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if epilogue not in binding.EPILOGUES:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    if epilogue in ("bias", "bias_gelu_tanh"):
        if bias is None:
            raise ValueError(f"epilogue {epilogue!r} needs a bias")
        _check(bias, "bias")
        if bias.shape != (N,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous [N] tensor")
    layout = _letter(x, "x") + _letter(W.t(), "W.T")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    elif out.shape != (M, N) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [M, N] tensor")
    lib = binding.load()
    wp, wb = _resolve_ws(workspace, "linear", M, N, K, layout, x.device)
    st = lib.mm_linear_ws(x.data_ptr(), W.data_ptr(), bias.data_ptr() if bias is not None else None,
                          out.data_ptr(), M, N, K, binding.LAYOUTS[layout],
                          binding.EPILOGUES[epilogue], wp, wb, _stream())
    binding.check(st, "mm_linear_ws")
    return out


def linear_preact(x: torch.Tensor, W: torch.Tensor, bias: Optional[torch.Tensor] = None,
                  epilogue: str = "bias_gelu_tanh", out: Optional[torch.Tensor] = None,
                  preact: Optional[torch.Tensor] = None):
    """LinearOp with two outputs from one kernel: preact = x @ W.T (+ bias) and
    out = GELU_tanh(preact), both bf16 [M, N]; epilogue gelu_tanh or
    bias_gelu_tanh.  Returns (out, preact)."""
    _check(x, "x")
    _check(W, "W")
    M, K = x.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if epilogue not in ("gelu_tanh", "bias_gelu_tanh"):
        raise ValueError("linear_preact needs epilogue gelu_tanh or bias_gelu_tanh")
    if epilogue == "bias_gelu_tanh":
        if bias is None:
            raise ValueError("epilogue 'bias_gelu_tanh' needs a bias")
        _check(bias, "bias")
        if bias.shape != (N,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous [N] tensor")
    layout = _letter(x, "x") + _letter(W.t(), "W.T")
    res = []
    for t, nm in ((out, "out"), (preact, "preact")):
        if t is None:
            t = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        elif t.shape != (M, N) or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous bf16 [M, N] tensor")
        res.append(t)
    out, preact = res
    lib = binding.load()
    st = lib.mm_linear_preact(x.data_ptr(), W.data_ptr(), bias.data_ptr() if bias is not None else None,
                              out.data_ptr(), preact.data_ptr(), M, N, K, binding.LAYOUTS[layout],
                              binding.EPILOGUES[epilogue], _stream())
    binding.check(st, "mm_linear_preact")
    return out, preact


def ffn_glu(x: torch.Tensor, W_gate: torch.Tensor, W_up: torch.Tensor, act: str = "silu",
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Horizontally fused FFN: out = act(x @ W_gate.T) * (x @ W_up.T), one kernel;
    x [M,K], W_gate and W_up [N,K] contiguous; act silu (Llama) or identity."""
    for t, nm in ((x, "x"), (W_gate, "W_gate"), (W_up, "W_up")):
        _check(t, nm)
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous 2-D tensor")
    M, K = x.shape
    N, K2 = W_gate.shape
    if K != K2 or W_up.shape != W_gate.shape:
        raise ValueError("shape mismatch between x, W_gate and W_up")
    if act not in binding.GLU_ACTS:
        raise ValueError(f"unknown activation {act!r}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    elif out.shape != (M, N) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [M, N] tensor")
    lib = binding.load()
    st = lib.mm_ffn_glu(x.data_ptr(), W_gate.data_ptr(), W_up.data_ptr(), out.data_ptr(), M, N, K,
                        binding.GLU_ACTS[act], _stream())
    binding.check(st, "mm_ffn_glu")
    return out


def ffn_swiglu(x: torch.Tensor, W_gate: torch.Tensor, W_up: torch.Tensor,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Llama FFN gate/up: SiLU(x @ W_gate.T) * (x @ W_up.T) in one kernel."""
    return ffn_glu(x, W_gate, W_up, "silu", out)


def _batched(t: torch.Tensor, name: str):
    """(entry layout letter, batch size, batch stride in elements) of a 3-D
    operand whose entries are contiguous or transposed-contiguous matrices;
    a batch dimension of size 1 or stride 0 broadcasts."""
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D [batch, rows, cols], got shape {tuple(t.shape)}")
    if t.shape[0] == 0:
        raise ValueError(f"{name} has an empty batch dimension")
    letter = _letter(t[0], name)
    stride = t.stride(0) if t.shape[0] > 1 else 0
    return letter, t.shape[0], stride


def _batch_count(*sizes: int) -> int:
    b = max(sizes)
    for s in sizes:
        if s not in (1, b):
            raise ValueError(f"batch sizes {sizes} do not broadcast")
    return b


def bmm(A: torch.Tensor, B: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Batched MatmulOp: out[b] = A[b] @ B[b] for A [batch, M, K], B [batch, K, N]
    (entries contiguous or transposed views; a batch dimension of 1, or an
    expanded one with stride 0, is broadcast).  One kernel for all entries."""
    _check(A, "A")
    _check(B, "B")
    la, ba, sa = _batched(A, "A")
    lb, bb, sb = _batched(B, "B")
    _, M, K = A.shape
    _, K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    batch = _batch_count(ba, bb)
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((batch, M, N), dtype=out_dtype, device=A.device)
    elif out.shape != (batch, M, N) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [batch, M, N] tensor of out_dtype")
    lib = binding.load()
    st = lib.mm_matmul_batched(A.data_ptr(), B.data_ptr(), out.data_ptr(), batch, M, N, K, sa, sb,
                               M * N, binding.LAYOUTS[la + lb],
                               binding.OUT_DTYPES["f32" if out_dtype == torch.float32 else "bf16"],
                               _stream())
    binding.check(st, "mm_matmul_batched")
    return out


def linear_batched(x: torch.Tensor, W: torch.Tensor, bias: Optional[torch.Tensor] = None,
                   epilogue: str = "none", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Batched LinearOp: out[b] = epi(x[b] @ W[b].T + bias) for x [batch, M, K] and
    W [batch, N, K] or [N, K] (one weight for every entry); bias [N] shared."""
    _check(x, "x")
    _check(W, "W")
    if W.dim() == 2:
        W = W.unsqueeze(0)
    lx, bx, sx = _batched(x, "x")
    lw, bw, sw = _batched(W.transpose(1, 2), "W.T")
    _, M, K = x.shape
    _, N, K2 = W.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if epilogue not in binding.EPILOGUES:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    if epilogue in ("bias", "bias_gelu_tanh"):
        if bias is None:
            raise ValueError(f"epilogue {epilogue!r} needs a bias")
        _check(bias, "bias")
        if bias.shape != (N,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous [N] tensor")
    batch = _batch_count(bx, bw)
    if out is None:
        out = torch.empty((batch, M, N), dtype=torch.bfloat16, device=x.device)
    elif out.shape != (batch, M, N) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [batch, M, N] tensor")
    lib = binding.load()
    st = lib.mm_linear_batched(x.data_ptr(), W.data_ptr(), bias.data_ptr() if bias is not None else None,
                               out.data_ptr(), batch, M, N, K, sx, sw, M * N,
                               binding.LAYOUTS[lx + lw], binding.EPILOGUES[epilogue], _stream())
    binding.check(st, "mm_linear_batched")
    return out
