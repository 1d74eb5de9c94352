"""GPU parity of the general layer (*_ex entry points: explicit mid, zero
padding to whole blocks, truncated output, bias) against the fp64
MonarchLinear-variant oracle. Bars as for the square/rectangular layer:
relative Frobenius error <= 1e-5 (fp32) and <= 2e-2 (bf16) per tensor."""
import sys

import numpy as np
import pytest

from oracle import monarch_linear as ML
from oracle.monarch_oracle import parity_error, rel_frobenius
from monarch_block_diagonal_amd import synthetic as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    from monarch_block_diagonal_amd import torch_api
    return torch_api


def tdt(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0").to(tdt(dtype))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(inp, out, mid, b1, b2, batch, dtype, seed):
    s = ML.general_sizes(inp, out, mid, b1, b2)
    w1 = S.draw(seed + 1, (b1, s["q1o"], s["q1i"]), "normal", 1.0 / s["q1i"], dtype)
    w2 = S.draw(seed + 2, (b2, s["q2o"], s["q2i"]), "normal", 1.0 / s["q2i"], dtype)
    x = S.draw(seed, (batch, inp), "normal", 1.0, dtype)
    dy = S.draw(seed + 3, (batch, out), "normal", 1.0, dtype)
    bias = S.draw(seed + 4, (out,), "normal", 0.25, dtype)
    return x, w1, w2, dy, bias


def check(api, inp, out, mid, b1, b2, batch, dtype, with_bias, relu, seed=7100):
    say(f"[linear] in={inp} out={out} mid={mid} b1={b1} b2={b2} batch={batch} {dtype} "
        f"bias={with_bias} relu={relu}")
    x, w1, w2, dy, bias = inputs(inp, out, mid, b1, b2, batch, dtype, seed)
    b = bias if with_bias else None
    act = 1 if relu else 0
    X, W1, W2 = dev(x, dtype), dev(w1, dtype), dev(w2, dtype)
    Bv = dev(bias, dtype) if with_bias else None
    y, z = api.monarch_forward_ex(X, W1, W2, out, Bv, act)
    torch.cuda.synchronize()
    y_ref = ML.forward_ex(x, w1, w2, inp, out, mid, b, relu)
    # row scales: the same results from the absolute values of every input
    ab = np.abs(b) if with_bias else None
    ys = ML.forward_ex(np.abs(x), np.abs(w1), np.abs(w2), inp, out, mid, ab, False)
    errs = {"y": parity_error(host(y), y_ref, ys)}
    # the GPU backward masks with the oracle's forward output, so both sides
    # mask the same entries
    mask = dev(y_ref, dtype) if relu else None
    dx, dw1, dw2, db = api.monarch_backward_ex(dev(dy, dtype), X, W1, W2, z, mask, with_bias, act)
    torch.cuda.synchronize()
    rx, r1, r2, rb = ML.backward_ex(dy, x, w1, w2, inp, out, mid, b, relu, y=y_ref)
    sx, s1, s2, sb = ML.backward_ex(np.abs(dy), np.abs(x), np.abs(w1), np.abs(w2), inp, out, mid,
                                    ab, relu, y=y_ref)
    errs.update(dx=parity_error(host(dx), rx, sx), dw1=parity_error(host(dw1), r1, s1),
                dw2=parity_error(host(dw2), r2, s2))
    if with_bias:
        errs["dbias"] = parity_error(host(db), rb, sb)
    say(f"[linear]   errors {errs}")
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


# (in, out, mid, nb1, nb2, batch)
SMALL = [
    (8, 16, 8, 2, 2, 9),
    (16, 8, 8, 2, 2, 33),
    (10, 7, 8, 4, 4, 5),
    (5, 13, 8, 4, 4, 70),
    (12, 20, 12, 3, 2, 17),
    (9, 6, 12, 4, 3, 130),
    (130, 200, 136, 8, 4, 300),       # several tiles, ragged, odd block sizes
    (1000, 333, 336, 3, 3, 257),      # q1i = 334, q2o = 111
    # at most 16 rows and K >= 128 (the skinny form): a K tail in both dtypes
    # with rows 8-byte aligned in bf16, bias and ReLU in its epilogue; and a
    # padded input whose blocks start off 16-byte boundaries in fp32
    (1000, 512, 512, 2, 2, 7),        # q1i = 500, q2i = 256
    (2500, 1024, 1024, 16, 16, 3),    # q1i = 157, the last block cut by the padding
]


@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("dtype,with_bias,relu", [("f32", True, True), ("bf16", True, False),
                                                  ("f32", False, False)])
def test_general_layer(api, shape, dtype, with_bias, relu):
    check(api, *shape, dtype, with_bias, relu)


@pytest.mark.parametrize("shape,dtype,with_bias", [
    ((768, 3072, 768, 4, 4, 1024), "bf16", True),     # MonarchLinear expanding branch (GPT-2 FFN up)
    ((3072, 768, 768, 4, 4, 512), "bf16", True),      # contracting branch (GPT-2 FFN down)
    ((2500, 1024, 1024, 16, 16, 100), "f32", False),  # q1i = 157, padded input
    ((1024, 1001, 1024, 4, 4, 1000), "f32", True),    # out not a multiple of the block count
])
def test_general_layer_larger(api, shape, dtype, with_bias):
    check(api, *shape, dtype, with_bias, False, seed=7200)


def test_page_rule_module(api):
    """MonarchLinear(in, out, nblocks) sizes its factors by the constructor
    rule and its autograd pass matches the oracle."""
    from monarch_block_diagonal_amd.torch_api import MonarchLinear
    torch.manual_seed(0)
    layer = MonarchLinear(50, 70, nblocks=4, bias=True, device="cuda:0")
    assert tuple(layer.w1.shape) == (4, 13, 13) and tuple(layer.w2.shape) == (4, 18, 13)
    x = torch.randn(37, 50, device="cuda:0", requires_grad=True)
    y = layer(x)
    dy = torch.randn_like(y)
    y.backward(dy)
    torch.cuda.synchronize()
    w1, w2, b = host(layer.w1), host(layer.w2), host(layer.bias)
    xx, dd = host(x), host(dy)
    y_ref = ML.forward_ex(xx, w1, w2, 50, 70, 52, b)
    rx, r1, r2, rb = ML.backward_ex(dd, xx, w1, w2, 50, 70, 52, b)
    for got, ref in ((y, y_ref), (x.grad, rx), (layer.w1.grad, r1), (layer.w2.grad, r2),
                     (layer.bias.grad, rb)):
        assert rel_frobenius(host(got), ref) <= 1e-5


def test_ex_equals_plain_entry_points_bitwise(api):
    """Whole blocks, mid = out, no bias: the same kernels and the same bits."""
    x, w1, w2, dy, _ = inputs(256, 512, 512, 4, 8, 300, "bf16", 7300)
    X, W1, W2, DY = dev(x, "bf16"), dev(w1, "bf16"), dev(w2, "bf16"), dev(dy, "bf16")
    y1, z1 = api.monarch_forward(X, W1, W2)
    y2, z2 = api.monarch_forward_ex(X, W1, W2, 512)
    a = api.monarch_backward(DY, X, W1, W2, z1)
    b = api.monarch_backward_ex(DY, X, W1, W2, z2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(z1, z2)
    for u, v in zip(a, b[:3]):
        assert torch.equal(u, v)


def test_batch_zero_and_one(api):
    x, w1, w2, dy, bias = inputs(10, 7, 8, 4, 4, 1, "f32", 7400)
    check(api, 10, 7, 8, 4, 4, 1, "f32", True, True, seed=7400)
    W1, W2 = dev(w1, "f32"), dev(w2, "f32")
    X0 = torch.empty((0, 10), device="cuda:0")
    y, z = api.monarch_forward_ex(X0, W1, W2, 7, dev(bias, "f32"))
    dx, dw1, dw2, db = api.monarch_backward_ex(torch.empty((0, 7), device="cuda:0"), X0, W1, W2,
                                               z, None, True)
    torch.cuda.synchronize()
    assert y.shape == (0, 7)
    assert not dw1.any() and not dw2.any() and not db.any()
