"""GPU parity of the DYAD-style layer against the fp64 oracle (relative
Frobenius error <= 1e-5 fp32, <= 2e-2 bf16, per tensor)."""
import sys

import numpy as np
import pytest

from oracle import dyad as D
from oracle.monarch_oracle import parity_error, rel_frobenius
from monarch_block_diagonal_amd import synthetic as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {"f32": 1e-5, "bf16": 2e-2}


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


@pytest.mark.parametrize("inp,out,nb,batch,dtype", [
    (16, 16, 4, 9, "f32"), (64, 32, 4, 300, "bf16"), (96, 192, 3, 70, "f32"),
    (48, 48, 6, 33, "bf16"), (8, 12, 1, 5, "f32"), (1024, 1024, 32, 1000, "bf16"),
    (768, 3072, 4, 512, "bf16"), (1000, 500, 10, 257, "f32"),
    # rows longer than one workgroup's LDS: the gathers take the tiled swap
    (32768, 256, 16, 6, "bf16"), (16000, 160, 16, 5, "f32"),
    # bf16 with 256 x 256 blocks: the block-diagonal kernel that keeps a
    # weight block in registers (one row, ragged tiles, several row ranges
    # per block, a short last range)
    (512, 512, 2, 1, "bf16"), (1024, 1024, 4, 100, "bf16"),
    (4096, 4096, 16, 1000, "bf16"), (2048, 2048, 8, 4133, "bf16"),
])
def test_dyad(api, inp, out, nb, batch, dtype):
    print(f"[dyad] in={inp} out={out} nb={nb} batch={batch} {dtype}", flush=True)
    qi, qo = inp // nb, out // nb
    wa = S.draw(9100, (nb, qo, qi), "normal", 0.5 / qi, dtype)
    wb = S.draw(9101, (nb, qo, qi), "normal", 0.5 / qi, dtype)
    x = S.draw(9102, (batch, inp), "normal", 1.0, dtype)
    dy = S.draw(9103, (batch, out), "normal", 1.0, dtype)
    X, WA, WB = dev(x, dtype), dev(wa, dtype), dev(wb, dtype)
    y = api.dyad_forward(X, WA, WB)
    dx, da, db = api.dyad_backward(dev(dy, dtype), X, WA, WB)
    torch.cuda.synchronize()
    rx, ra, rb = D.backward(dy, x, wa, wb, inp, out)
    # row scales: the same results from the absolute values of every input
    A = np.abs
    ys = D.forward(A(x), A(wa), A(wb), inp, out)
    sx, sa, sb = D.backward(A(dy), A(x), A(wa), A(wb), inp, out)
    errs = {"y": parity_error(host(y), D.forward(x, wa, wb, inp, out), ys),
            "dx": parity_error(host(dx), rx, sx), "dA": parity_error(host(da), ra, sa),
            "dB": parity_error(host(db), rb, sb)}
    print(f"[dyad]   errors {errs}", flush=True)
    sys.stdout.flush()
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)
