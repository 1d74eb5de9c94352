"""GPU parity of the dense -> Monarch projection (monarch_project) against the
projection oracle. Inputs: seeded near-Monarch matrices (a random Monarch
matrix plus small dense noise, the use the pages describe: fitting Monarch
factors to a trained dense layer) and exact Monarch matrices. Factors are
compared slice by slice through their outer products (the fit is unique; the
sign rule is checked separately where the largest entry is well separated)."""
import sys

import numpy as np
import pytest

import oracle as O
from oracle import monarch_projection as PJ
from monarch_block_diagonal_amd import synthetic as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def api():
    from monarch_block_diagonal_amd import torch_api
    return torch_api


def near_monarch(inp, out, b1, b2, noise, seed):
    s = O.derive_sizes(inp, out, b1, b2)
    w1 = S.draw(seed, (b1, s["q1o"], s["q1i"]), "normal", 1.0 / s["q1i"], "f32").astype(np.float64)
    w2 = S.draw(seed + 1, (b2, s["q2o"], s["q2i"]), "normal", 1.0 / s["q2i"], "f32").astype(np.float64)
    m = O.monarch_matrix(w1, w2, inp, out)
    if noise:
        m = m + noise * np.sqrt(np.mean(m * m)) * S.draw(seed + 2, (out, inp), "normal", 1.0, "f32")
    return m


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def slice_products(w1, w2):
    """[b2, b1, q2o, q1i] outer products L[g, :, r] R[r, g, :]."""
    return np.einsum("gpr,rgs->grps", w2, w1)


SHAPES = [(16, 16, 4, 4), (12, 8, 2, 4), (64, 64, 8, 8), (1024, 1024, 32, 32), (96, 6, 2, 3),
          (4096, 4096, 64, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_project_near_monarch(api, shape, dtype):
    inp, out, b1, b2 = shape
    m = near_monarch(inp, out, b1, b2, 1e-3, seed=3000 + inp + out)
    if dtype == "bf16":
        m = S.round_to_bf16(m.astype(np.float32)).astype(np.float64)
    r1, r2 = PJ.project(m, inp, out, b1, b2)
    w1, w2 = api.monarch_project(to_dev(m, dtype), b1, b2, iters=32)
    torch.cuda.synchronize()
    g1, g2 = host(w1), host(w2)
    e_prod = O.rel_frobenius(slice_products(g1, g2), slice_products(r1, r2))
    e_mat = O.rel_frobenius(O.monarch_matrix(g1, g2, inp, out), O.monarch_matrix(r1, r2, inp, out))
    e1, e2 = O.rel_frobenius(g1, r1), O.rel_frobenius(g2, r2)
    say(f"[parity] project {shape} {dtype}: slices {e_prod:.2e} matrix {e_mat:.2e} "
        f"w1 {e1:.2e} w2 {e2:.2e}")
    assert e_prod <= TOL[dtype] and e_mat <= TOL[dtype]
    # factors themselves (split and sign rule) agree as well
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype]


@pytest.mark.parametrize("shape", [(16, 16, 4, 4), (1024, 1024, 32, 32), (12, 8, 2, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_project_reproduces_monarch_input(api, shape):
    """An exact Monarch matrix is its own projection (one iteration is enough)."""
    inp, out, b1, b2 = shape
    m = near_monarch(inp, out, b1, b2, 0.0, seed=4000 + inp)
    w1, w2 = api.monarch_project(to_dev(m, "f32"), b1, b2, iters=1)
    torch.cuda.synchronize()
    mh = O.monarch_matrix(host(w1), host(w2), inp, out)
    e = O.rel_frobenius(mh, m)
    say(f"[parity] project exact {shape}: {e:.2e}")
    assert e <= TOL["f32"]


def test_project_full_size_sampled(api):
    """n = 16384 with 128 x 128 blocks (16384 slices of 128 x 128), bf16, in
    the launch configuration the benchmark times; sampled slices against the
    oracle's fit of the same slices."""
    inp = out = 16384
    b1 = b2 = 128
    g = torch.Generator(device="cuda:0")
    g.manual_seed(777)
    w1 = torch.randn((b1, b2, 128), generator=g, device="cuda:0") / 128 ** 0.5
    w2 = torch.randn((b2, 128, b1), generator=g, device="cuda:0") / 128 ** 0.5
    # dense M from the Monarch definition, slice by slice on the device
    # (M[p*b2 + g, r*q1i + s] = L[g, p, r] R[r, g, s]) plus 1e-3 relative noise
    mt = torch.einsum("gpr,rgs->pgrs", w2, w1).reshape(out, inp)
    mt = mt + 1e-3 * mt.std() * torch.randn(mt.shape, generator=g, device="cuda:0")
    m = mt.to(torch.bfloat16)
    del mt
    p1, p2 = api.monarch_project(m, b1, b2, iters=32)
    torch.cuda.synchronize()
    gs = [(0, 0), (5, 77), (127, 127), (64, 3)]
    mh = m.float()
    for gg, rr in gs:
        sl = host(mh[gg::b2, rr * 128:(rr + 1) * 128])
        lv, rv = PJ.fit_slice(sl)
        ref = np.outer(lv, rv)
        got = np.outer(host(p2[gg, :, rr]), host(p1[rr, gg, :]))
        e = O.rel_frobenius(got, ref)
        say(f"[parity] project full size slice ({gg},{rr}): {e:.2e}")
        assert e <= TOL["bf16"]
