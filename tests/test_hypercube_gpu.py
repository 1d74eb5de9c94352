"""GPU parity of the k-factor (hypercube) layer against the fp64 oracle.
Bars: relative Frobenius error <= 1e-5 (fp32) and <= 2e-2 (bf16) for y, dx
and every round's weight gradient; bit-exact for identity weights."""
import sys

import numpy as np
import pytest

from oracle import monarch_hypercube as H
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


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")
    return t if dtype == "f32" else t.to(torch.bfloat16)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(api, dims, batch, dtype, seed=8100):
    n = int(np.prod(dims))
    say(f"[hyper] dims={dims} batch={batch} {dtype}")
    ws = [S.draw(seed + 1 + j, s, "normal", 1.0 / s[2], dtype)
          for j, s in enumerate(H.weight_shapes(dims))]
    x = S.draw(seed, (batch, n), "normal", 1.0, dtype)
    dy = S.draw(seed + 9, (batch, n), "normal", 1.0, dtype)
    X, DY, W = dev(x, dtype), dev(dy, dtype), [dev(w, dtype) for w in ws]
    y, saved = api.hyper_forward(X, W, dims)
    dx, dws = api.hyper_backward(DY, X, W, saved, dims)
    torch.cuda.synchronize()
    y_ref = H.forward_fibers(x, ws, dims)
    rx, rws = H.backward_fibers(dy, x, ws, dims)
    # row scales: the same results from the absolute values of every input
    aws = [np.abs(w) for w in ws]
    ys = H.forward_fibers(np.abs(x), aws, dims)
    sx, sws = H.backward_fibers(np.abs(dy), np.abs(x), aws, dims)
    errs = {"y": parity_error(host(y), y_ref, ys), "dx": parity_error(host(dx), rx, sx)}
    for j, (g, r, sc) in enumerate(zip(dws, rws, sws)):
        errs[f"dw{j + 1}"] = parity_error(host(g), r, sc)
    say(f"[hyper]   errors {errs}")
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


@pytest.mark.parametrize("dims,batch,dtype", [
    ((2, 3, 4), 5, "f32"), ((4, 8), 33, "bf16"), ((8, 4, 2), 40, "f32"),
    ((16, 2, 2, 3), 7, "bf16"), ((6,), 9, "f32"), ((32, 16), 300, "bf16"),
    ((16, 16, 16), 130, "f32"), ((5, 7, 3), 257, "f32"),
    # bf16 fibers of 24 with a partial segment (15 fibers: 8 + 7) and weight
    # gradients over several row chunks, the last one ragged
    ((24, 5, 3), 1000, "bf16"), ((3, 16, 32), 1500, "bf16"),
    # bf16 rounds fused with their layout swap: several arrays per row
    # ((4, 16, 8): forward round 1), an axis after the pair ((2, 24, 8, 2)),
    # the backward direction ((8, 32, 2)), batches not a multiple of 32
    ((4, 16, 8), 77, "bf16"), ((2, 24, 8, 2), 100, "bf16"), ((8, 32, 2), 45, "bf16"),
    # bf16 round 0 joined with the transposes: a partial chunk of 40 fibers,
    # 72 fibers (64 + 8), three axes
    ((16, 40), 77, "bf16"), ((24, 72), 33, "bf16"), ((32, 8, 3), 100, "bf16"),
])
def test_hyper_small(api, dims, batch, dtype):
    check(api, dims, batch, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hyper_large_arrays(api, dtype):
    """38400 units: the transposes and the first layout swap exceed one
    workgroup's LDS and take the 32 x 32-tile swap kernel (partial tiles on
    both axes)."""
    check(api, (64, 20, 30), 6, dtype, seed=8300)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hyper_page_lattice(api, dtype):
    """The page's 12288-unit lattice 16 x 24 x 32."""
    check(api, (16, 24, 32), 256, dtype, seed=8200)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hyper_identity_is_exact(api, dtype):
    dims = (8, 4, 6)
    n = int(np.prod(dims))
    ws = [np.broadcast_to(np.eye(d), s).copy() for d, s in zip(dims, H.weight_shapes(dims))]
    x = S.draw(8300, (70, n), "normal", 1.0, dtype)
    X = dev(x, dtype)
    y, saved = api.hyper_forward(X, [dev(w, dtype) for w in ws], dims)
    torch.cuda.synchronize()
    assert torch.equal(y, X)
