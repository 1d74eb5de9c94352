"""Tensor-level helpers over the C ABI: PyTorch allocates device memory and
supplies the stream; the library's kernels do all the arithmetic.

    y, z = monarch_forward(x, w1, w2)              # x [B, in], w1 [b1, q1o, q1i], w2 [b2, q2o, q2i]
    dx, dw1, dw2 = monarch_backward(dy, x, w1, w2, z)

MonarchLinearFunction wraps the pair as an autograd function, so the operator
can stand in for a dense linear layer. The *_ex helpers and the MonarchLinear
module take the general layer (any in/out, zero-padded to whole blocks, an
explicit intermediate width, optional bias).
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


def _expect(t, shape, name: str):
    """Raise ValueError unless tensor t (if given) has exactly this shape; the
    kernels derive every extent from the sizes passed to the library, so a
    tensor of another shape would be read or written out of its bounds."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def problem_of(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor):
    """(in_features, out_features, nblocks1, nblocks2, batch) from tensor shapes,
    after checking w1 == [b1, out/b1, in/b1] and w2 == [b2, out/b2, out/b2]
    (mid = out)."""
    if x.dim() != 2 or w1.dim() != 3 or w2.dim() != 3:
        raise ValueError("x must be [batch, in], w1 [b1, q1o, q1i], w2 [b2, q2o, q2i]")
    nb1, nb2 = int(w1.shape[0]), int(w2.shape[0])
    fi, fo, b = int(x.shape[1]), nb2 * int(w2.shape[1]), int(x.shape[0])
    if nb1 <= 0 or nb2 <= 0 or fi % nb1 or fo % nb1:
        raise ValueError(f"in={fi} and out={fo} must be divisible by nblocks1={nb1}")
    _expect(w1, (nb1, fo // nb1, fi // nb1), "w1")
    _expect(w2, (nb2, fo // nb2, fo // nb2), "w2")
    return fi, fo, nb1, nb2, b


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
    fi, fo, nb1, nb2, b = problem_of(x, w1, w2)
    _check(x, w1, w2)
    y = torch.empty((b, fo), dtype=x.dtype, device=x.device)
    z = torch.empty((b, fo), dtype=x.dtype, device=x.device)
    B.monarch_fwd(x, w1, w2, y, z, fi, fo, nb1, nb2, b, dtype_code(x), act, stream)
    return y, z


def monarch_backward(dy, x, w1, w2, z, y=None, act: int = B.ACT_NONE, stream=None,
                     workspace: torch.Tensor | None = None):
    fi, fo, nb1, nb2, b = problem_of(x, w1, w2)
    for t, name in ((dy, "dy"), (z, "z"), (y, "y")):
        _expect(t, (b, fo), name)
    if act == B.ACT_RELU and y is None:
        raise ValueError("the ReLU backward needs the forward output y")
    _check(dy, x, w1, w2, z, y)
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


def monarch_project(m, nblocks1: int, nblocks2: int, max_steps: int = 256, stream=None,
                    with_status: bool = False):
    """Nearest Monarch factors (w1 [b1, b2, in/b1], w2 [b2, out/b2, b1]) of a
    dense [out, in] matrix; needs out = nblocks1 * nblocks2. With with_status,
    also returns the int32 [b1 * b2] per-slice status (element r*b2 + g for
    slice (g, r)): the products with AᵀA it used when converged, else 0."""
    _check(m)
    if m.dim() != 2:
        raise ValueError("m must be [out, in]")
    fo, fi = m.shape
    if nblocks1 <= 0 or nblocks2 <= 0 or fi % nblocks1 or fo % nblocks2:
        raise ValueError("block counts must divide the matrix dimensions")
    w1 = torch.empty((nblocks1, nblocks2, fi // nblocks1), dtype=m.dtype, device=m.device)
    w2 = torch.empty((nblocks2, fo // nblocks2, nblocks1), dtype=m.dtype, device=m.device)
    conv = torch.empty((nblocks1 * nblocks2,), dtype=torch.int32, device=m.device)
    B.monarch_project(m, w1, w2, fi, fo, nblocks1, nblocks2, dtype_code(m), max_steps, conv,
                      stream)
    return (w1, w2, conv) if with_status else (w1, w2)


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


def ex_problem(x, w1, w2, out_features: int, bias=None):
    """(in, out, mid, nb1, nb2, batch) of the general layer from tensor shapes,
    after checking w1 == [b1, mid/b1, ceil(in/b1)], w2 == [b2, ceil(out/b2),
    mid/b2] and bias == [out]."""
    if x.dim() != 2 or w1.dim() != 3 or w2.dim() != 3:
        raise ValueError("x must be [batch, in], w1 [b1, q1o, q1i], w2 [b2, q2o, q2i]")
    nb1, q1o = int(w1.shape[0]), int(w1.shape[1])
    nb2 = int(w2.shape[0])
    mid = nb1 * q1o
    fi, fo, b = int(x.shape[1]), int(out_features), int(x.shape[0])
    if nb1 <= 0 or nb2 <= 0 or fi <= 0 or fo <= 0 or mid % nb2:
        raise ValueError(f"mid={mid} must be divisible by nblocks2={nb2}; sizes must be positive")
    _expect(w1, (nb1, q1o, _cdiv(fi, nb1)), "w1")
    _expect(w2, (nb2, _cdiv(fo, nb2), mid // nb2), "w2")
    if bias is not None and (bias.dim() != 1 or bias.numel() != fo):
        raise ValueError(f"bias has shape {tuple(bias.shape)}, expected ({fo},)")
    return fi, fo, mid, nb1, nb2, b


def monarch_forward_ex(x, w1, w2, out_features: int, bias=None, act: int = B.ACT_NONE,
                       stream=None):
    """y = act(pad(x) · Mᵀ truncated to out_features + bias); returns (y, z)."""
    fi, fo, mid, nb1, nb2, b = ex_problem(x, w1, w2, out_features, bias)
    _check(x, w1, w2, bias)
    y = torch.empty((b, fo), dtype=x.dtype, device=x.device)
    z = torch.empty((b, mid), dtype=x.dtype, device=x.device)
    B.monarch_fwd_ex(x, w1, w2, bias, y, z, fi, fo, mid, nb1, nb2, b, dtype_code(x), act, stream)
    return y, z


def monarch_backward_ex(dy, x, w1, w2, z, y=None, with_bias: bool = False,
                        act: int = B.ACT_NONE, stream=None):
    """(dx, dw1, dw2, dbias or None) of the general layer."""
    if dy.dim() != 2:
        raise ValueError("dy must be [batch, out]")
    fi, fo, mid, nb1, nb2, b = ex_problem(x, w1, w2, dy.shape[1])
    _expect(dy, (b, fo), "dy")
    _expect(y, (b, fo), "y")
    _expect(z, (b, mid), "z")
    if act == B.ACT_RELU and y is None:
        raise ValueError("the ReLU backward needs the forward output y")
    _check(dy, x, w1, w2, z, y)
    code = dtype_code(x)
    dx = torch.empty_like(x)
    dw1 = torch.empty_like(w1)
    dw2 = torch.empty_like(w2)
    db = torch.empty((fo,), dtype=x.dtype, device=x.device) if with_bias else None
    need = B.monarch_bwd_ex_workspace_bytes(fi, fo, mid, nb1, nb2, b, code, with_bias)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    B.monarch_bwd_ex(dy, x, w1, w2, z, y, dx, dw1, dw2, db, ws, need, fi, fo, mid, nb1, nb2, b,
                     code, act, stream)
    return dx, dw1, dw2, db


class MonarchLinearExFunction(torch.autograd.Function):
    """y = act(pad(x) · Mᵀ truncated to out_features + bias)."""

    @staticmethod
    def forward(ctx, x, w1, w2, bias, out_features: int, act: int = B.ACT_NONE):
        x, w1, w2 = x.contiguous(), w1.contiguous(), w2.contiguous()
        bias = bias.contiguous() if bias is not None else None
        y, z = monarch_forward_ex(x, w1, w2, out_features, bias, act)
        ctx.act = act
        ctx.with_bias = bias is not None
        ctx.save_for_backward(x, w1, w2, z, y if act == B.ACT_RELU else None)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w1, w2, z, y = ctx.saved_tensors
        dx, dw1, dw2, db = monarch_backward_ex(dy.contiguous(), x, w1, w2, z, y, ctx.with_bias,
                                               ctx.act)
        return dx, dw1, dw2, db, None, None


class MonarchLinear(torch.nn.Module):
    """Drop-in for a dense linear layer with the MonarchLinear sizes of the
    "Definition C.3" thread of the scatterbrain issues page: block sizes
    ceil(in/nblocks) and ceil(out/nblocks), intermediate width in_ext for an
    expanding layer and out_ext otherwise; the input is zero-padded to whole
    blocks and the output keeps the first out_features. Optional bias and
    fused ReLU (act)."""

    def __init__(self, in_features: int, out_features: int, nblocks: int = 4, bias: bool = True,
                 act: int = B.ACT_NONE, device=None, dtype=torch.float32):
        super().__init__()
        self.in_features, self.out_features, self.nblocks, self.act = (
            in_features, out_features, nblocks, act)
        mid = B.monarch_linear_mid(in_features, out_features, nblocks)
        q1i = -(-in_features // nblocks)
        q2o = -(-out_features // nblocks)
        self.mid = mid
        self.w1 = torch.nn.Parameter(torch.empty((nblocks, mid // nblocks, q1i), device=device,
                                                 dtype=dtype))
        self.w2 = torch.nn.Parameter(torch.empty((nblocks, q2o, mid // nblocks), device=device,
                                                 dtype=dtype))
        self.bias = (torch.nn.Parameter(torch.empty(out_features, device=device, dtype=dtype))
                     if bias else None)
        self.reset_parameters()

    @torch.no_grad()
    def reset_parameters(self):
        # each factor block is a small dense layer: uniform(+-1/sqrt(fan_in))
        for w in (self.w1, self.w2):
            bound = w.shape[2] ** -0.5
            w.uniform_(-bound, bound)
        if self.bias is not None:
            self.bias.uniform_(-self.in_features ** -0.5, self.in_features ** -0.5)

    def forward(self, x):
        shape = x.shape
        y = MonarchLinearExFunction.apply(x.reshape(-1, shape[-1]), self.w1, self.w2, self.bias,
                                          self.out_features, self.act)
        return y.reshape(*shape[:-1], self.out_features)


def _hyper_shapes(x, ws, dims):
    """Check x == [batch, N] and ws[j] == [N/n_j, n_j, n_j] (N = prod dims)."""
    dims = [int(d) for d in dims]
    if x.dim() != 2 or len(ws) != len(dims) or not dims or min(dims) <= 0:
        raise ValueError("x must be [batch, N] with one weight tensor per lattice axis")
    n = 1
    for d in dims:
        n *= d
    _expect(x, (x.shape[0], n), "x")
    for j, (w, d) in enumerate(zip(ws, dims)):
        _expect(w, (n // d, d, d), f"ws[{j}]")
    return int(x.shape[0]), n


def hyper_forward(x, ws, dims, stream=None):
    """k-factor (hypercube) layer: x [batch, N], ws[j] [N/n_j, n_j, n_j];
    returns (y, saved)."""
    b, n = _hyper_shapes(x, ws, dims)
    _check(x, *ws)
    saved = torch.empty((max(B.monarch_hyper_saved_elems(dims, b), 1),), dtype=x.dtype,
                        device=x.device)
    y = torch.empty_like(x)
    B.monarch_hyper_fwd(x, ws, y, saved, dims, b, dtype_code(x), stream)
    return y, saved


def hyper_backward(dy, x, ws, saved, dims, stream=None):
    """(dx, [dw_j]) of the hypercube layer."""
    b, n = _hyper_shapes(x, ws, dims)
    _expect(dy, (b, n), "dy")
    if saved.numel() < B.monarch_hyper_saved_elems(dims, b):
        raise ValueError("saved is smaller than the forward pass writes")
    _check(dy, x, *ws)
    code = dtype_code(x)
    dx = torch.empty_like(x)
    dws = [torch.empty_like(w) for w in ws]
    need = B.monarch_hyper_bwd_workspace_bytes(dims, b, code)
    ws_buf = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    B.monarch_hyper_bwd(dy, x, ws, saved, dx, dws, ws_buf, need, dims, b, code, stream)
    return dx, dws


def _dyad_shapes(x, wa, wb):
    """Check wb == wa == [nb, qo, qi] and x == [batch, nb*qi]."""
    if x.dim() != 2 or wa.dim() != 3:
        raise ValueError("x must be [batch, in], wa and wb [nb, out/nb, in/nb]")
    nb, qo, qi = (int(v) for v in wa.shape)
    _expect(wb, (nb, qo, qi), "wb")
    _expect(x, (x.shape[0], nb * qi), "x")
    return nb, qo, qi, int(x.shape[0])


def dyad_forward(x, wa, wb, stream=None):
    """DYAD-style layer: y = x · (BD(A) + Q·BD(B)·P)ᵀ; wa, wb [nb, out/nb, in/nb]."""
    nb, qo, qi, b = _dyad_shapes(x, wa, wb)
    _check(x, wa, wb)
    y = torch.empty((b, nb * qo), dtype=x.dtype, device=x.device)
    need = B.monarch_dyad_fwd_workspace_bytes(x.shape[1], nb * qo, nb, b, dtype_code(x))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    B.monarch_dyad_fwd(x, wa, wb, y, ws, need, x.shape[1], nb * qo, nb, b, dtype_code(x), stream)
    return y


def dyad_backward(dy, x, wa, wb, stream=None):
    """(dx, dwa, dwb) of the DYAD-style layer."""
    nb, qo, qi, b = _dyad_shapes(x, wa, wb)
    _expect(dy, (b, nb * qo), "dy")
    _check(dy, x, wa, wb)
    code = dtype_code(x)
    dx, dwa, dwb = torch.empty_like(x), torch.empty_like(wa), torch.empty_like(wb)
    need = B.monarch_dyad_bwd_workspace_bytes(x.shape[1], nb * qo, nb, b, code)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    B.monarch_dyad_bwd(dy, x, wa, wb, dx, dwa, dwb, ws, need, x.shape[1], nb * qo, nb, b, code,
                       stream)
    return dx, dwa, dwb
