"""Tensor-level helpers over the C ABI: PyTorch allocates device memory and
supplies the stream; the library's kernels do all the arithmetic.

    y, z = monarch_forward(x, w1, w2)              # x [B, in], w1 [b1, q1o, q1i], w2 [b2, q2o, q2i]
    dx, dw1, dw2 = monarch_backward(dy, x, w1, w2, z)

MonarchLinearFunction wraps the pair as an autograd function, so the operator
can stand in for a dense linear layer.
"""
from __future__ import annotations

import torch

from . import binding as B


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return B.F32
    if t.dtype == torch.bfloat16:
        return B.BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def problem_of(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor):
    """(in_features, out_features, nblocks1, nblocks2, batch) from tensor shapes."""
    if x.dim() != 2 or w1.dim() != 3 or w2.dim() != 3:
        raise ValueError("x must be [batch, in], w1 [b1, q1o, q1i], w2 [b2, q2o, q2i]")
    nb1, q1o, q1i = w1.shape
    nb2, q2o, q2i = w2.shape
    return x.shape[1], nb2 * q2o, nb1, nb2, x.shape[0]


def _check(*ts):
    dt = ts[0].dtype
    for t in ts:
        if t is None:
            continue
        if t.dtype != dt:
            raise TypeError("all tensors must share one dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")


def monarch_forward(x, w1, w2, act: int = B.ACT_NONE, stream=None):
    _check(x, w1, w2)
    fi, fo, nb1, nb2, b = problem_of(x, w1, w2)
    y = torch.empty((b, fo), dtype=x.dtype, device=x.device)
    z = torch.empty((b, fo), dtype=x.dtype, device=x.device)
    B.monarch_fwd(x, w1, w2, y, z, fi, fo, nb1, nb2, b, dtype_code(x), act, stream)
    return y, z


def monarch_backward(dy, x, w1, w2, z, y=None, act: int = B.ACT_NONE, stream=None,
                     workspace: torch.Tensor | None = None):
    _check(dy, x, w1, w2, z, y)
    fi, fo, nb1, nb2, b = problem_of(x, w1, w2)
    code = dtype_code(x)
    dx = torch.empty_like(x)
    dw1 = torch.empty_like(w1)
    dw2 = torch.empty_like(w2)
    need = B.monarch_bwd_workspace_bytes(fi, fo, nb1, nb2, b, code)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    B.monarch_bwd(dy, x, w1, w2, z, y, dx, dw1, dw2, workspace, need, fi, fo, nb1, nb2, b, code,
                  act, stream)
    return dx, dw1, dw2


def monarch_project(m, nblocks1: int, nblocks2: int, iters: int = 32, stream=None):
    """Nearest Monarch factors (w1 [b1, b2, in/b1], w2 [b2, out/b2, b1]) of a
    dense [out, in] matrix; needs out = nblocks1 * nblocks2."""
    _check(m)
    if m.dim() != 2:
        raise ValueError("m must be [out, in]")
    fo, fi = m.shape
    if nblocks1 <= 0 or nblocks2 <= 0 or fi % nblocks1 or fo % nblocks2:
        raise ValueError("block counts must divide the matrix dimensions")
    w1 = torch.empty((nblocks1, nblocks2, fi // nblocks1), dtype=m.dtype, device=m.device)
    w2 = torch.empty((nblocks2, fo // nblocks2, nblocks1), dtype=m.dtype, device=m.device)
    B.monarch_project(m, w1, w2, fi, fo, nblocks1, nblocks2, dtype_code(m), iters, stream)
    return w1, w2


class MonarchLinearFunction(torch.autograd.Function):
    """y = act(x · Mᵀ) with M the Monarch matrix of (w1, w2); no bias."""

    @staticmethod
    def forward(ctx, x, w1, w2, act: int = B.ACT_NONE):
        x, w1, w2 = x.contiguous(), w1.contiguous(), w2.contiguous()
        y, z = monarch_forward(x, w1, w2, act)
        ctx.act = act
        ctx.save_for_backward(x, w1, w2, z, y if act == B.ACT_RELU else None)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w1, w2, z, y = ctx.saved_tensors
        dx, dw1, dw2 = monarch_backward(dy.contiguous(), x, w1, w2, z, y, ctx.act)
        return dx, dw1, dw2, None
