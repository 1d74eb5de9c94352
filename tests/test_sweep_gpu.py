"""Seeded random sweep of layer shapes against the fp64 oracle (GPU).

Covers the three paths with shapes the hand-picked cases do not: random
block counts and block sizes, padded inputs and truncated outputs, bias,
ReLU and ragged batches on the generic path (small layers, bf16 layers of
256-1536 features that take the large tiles, bf16 layers whose stage-1
blocks take the register-resident block-diagonal form, and batches of at
most 16 rows with long stage-1 blocks); random batches on the
fused 32x32-block and square 128x128-block paths. The shapes come from a fixed
seed, so every run checks the same cases; the ids name them.
"""
import math
import random
import sys

import numpy as np
import pytest

import oracle as O
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


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")
    return t if dtype == "f32" else t.to(torch.bfloat16)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _general_cases():
    rng = random.Random(20221203)
    cases = []
    for _ in range(24):
        b1, b2 = rng.randint(1, 8), rng.randint(1, 8)
        lcm = b1 * b2 // math.gcd(b1, b2)
        mid = lcm * rng.randint(1, max(1, 256 // lcm))
        cases.append((rng.randint(1, 300), rng.randint(1, 300), mid, b1, b2, rng.randint(1, 300),
                      rng.choice(["f32", "bf16"]), rng.random() < 0.5, rng.random() < 0.5))
    return cases


def _square_cases():
    rng = random.Random(20221204)
    cases = []
    for n, nb in [(256, 8), (512, 16), (1024, 32), (1024, 32), (4096, 32), (4096, 32)]:
        batch = rng.randint(1, 2000 if n <= 1024 else 300)
        cases.append((n, nb, batch, rng.random() < 0.5))
    return cases


def _large_cases():
    # bf16 layers wide enough for the 256 x 256 and 256 x 192 tiles, with
    # ragged rows, columns and K and batch-split weight gradients
    rng = random.Random(20221205)
    cases = []
    for _ in range(12):
        b1, b2 = rng.randint(1, 4), rng.randint(1, 4)
        lcm = b1 * b2 // math.gcd(b1, b2)
        mid = lcm * rng.randint(max(1, 256 // lcm), 1536 // lcm)
        cases.append((rng.randint(256, 1536), rng.randint(256, 1536), mid, b1, b2,
                      rng.randint(256, 1500), "bf16", rng.random() < 0.3, rng.random() < 0.3))
    return cases


def _blockdiag_cases():
    # bf16 layers whose stage-1 blocks have 192 or 256 inputs and a multiple
    # of 256 outputs (the register-resident block-diagonal form, one to three
    # column slices, with or without stage 2's column split), sometimes with
    # a padded input (the last block cut: the tiled form instead)
    rng = random.Random(20221206)
    cases = []
    for _ in range(8):
        b1 = rng.randint(1, 4)
        q1i, q1o = rng.choice([192, 256]), 256 * rng.randint(1, 3)
        mid = b1 * q1o
        b2 = rng.choice([d for d in (1, 2, 3, 4, 6, 8, 16, 64) if mid % d == 0])
        inp = b1 * q1i - (rng.randint(1, 40) if rng.random() < 0.25 else 0)
        cases.append((inp, rng.randint(64, 1536), mid, b1, b2, rng.randint(1, 700), "bf16",
                      rng.random() < 0.3, rng.random() < 0.3))
    return cases


def _skinny_cases():
    # at most 16 rows with stage-1 blocks of 128 or more inputs (K split over
    # the waves of a workgroup), odd and even strides, K tails
    rng = random.Random(20221207)
    cases = []
    for _ in range(8):
        b1, b2 = rng.randint(1, 4), rng.randint(1, 4)
        lcm = b1 * b2 // math.gcd(b1, b2)
        mid = lcm * rng.randint(max(1, 64 // lcm), max(2, 768 // lcm))
        cases.append((b1 * rng.randint(128, 700), rng.randint(16, 600), mid, b1, b2,
                      rng.randint(1, 16), rng.choice(["f32", "bf16"]), rng.random() < 0.5,
                      rng.random() < 0.5))
    return cases


GENERAL = _general_cases()
SQUARE = _square_cases()
LARGE = _large_cases()
BLOCKDIAG = _blockdiag_cases()
SKINNY = _skinny_cases()


@pytest.mark.parametrize("case", GENERAL + LARGE + BLOCKDIAG + SKINNY, ids=lambda c: "in%d-out%d-mid%d-b%dx%d-B%d-%s-bias%d-relu%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[8]))
def test_sweep_general(api, case):
    inp, out, mid, b1, b2, batch, dtype, with_bias, relu = case
    say(f"[sweep] {case}")
    seed = 9000 + inp * 7 + out * 3 + batch
    s = ML.general_sizes(inp, out, mid, b1, b2)
    w1 = S.draw(seed + 1, (b1, s["q1o"], s["q1i"]), "normal", 1.0 / s["q1i"], dtype)
    w2 = S.draw(seed + 2, (b2, s["q2o"], s["q2i"]), "normal", 1.0 / s["q2i"], dtype)
    x = S.draw(seed, (batch, inp), "normal", 1.0, dtype)
    dy = S.draw(seed + 3, (batch, out), "normal", 1.0, dtype)
    bias = S.draw(seed + 4, (out,), "normal", 0.25, dtype) if with_bias else None
    act = 1 if relu else 0
    X, W1, W2 = dev(x, dtype), dev(w1, dtype), dev(w2, dtype)
    y, z = api.monarch_forward_ex(X, W1, W2, out, dev(bias, dtype) if with_bias else None, act)
    torch.cuda.synchronize()
    y_ref = ML.forward_ex(x, w1, w2, inp, out, mid, bias, relu)
    # the GPU backward masks with the oracle's forward output
    mask = dev(y_ref, dtype) if relu else None
    dx, dw1, dw2, db = api.monarch_backward_ex(dev(dy, dtype), X, W1, W2, z, mask, with_bias, act)
    torch.cuda.synchronize()
    rx, r1, r2, rb = ML.backward_ex(dy, x, w1, w2, inp, out, mid, bias, relu, y=y_ref)
    # row scales: the same results from the absolute values of every input
    ab = np.abs(bias) if with_bias else None
    ys = ML.forward_ex(np.abs(x), np.abs(w1), np.abs(w2), inp, out, mid, ab, False)
    sx, s1, s2, sb = ML.backward_ex(np.abs(dy), np.abs(x), np.abs(w1), np.abs(w2), inp, out, mid,
                                    ab, relu, y=y_ref)
    errs = {"y": parity_error(host(y), y_ref, ys), "dx": parity_error(host(dx), rx, sx),
            "dw1": parity_error(host(dw1), r1, s1), "dw2": parity_error(host(dw2), r2, s2)}
    if with_bias:
        errs["dbias"] = parity_error(host(db), rb, sb)
    say(f"[sweep]   errors {errs}")
    for k, e in errs.items():
        assert e <= TOL[dtype], (case, k, e)


@pytest.mark.parametrize("case", SQUARE, ids=lambda c: "n%d-nb%d-B%d-relu%d" % c)
def test_sweep_square_paths(api, case):
    """bf16 square layers with 32x32 blocks (fused path) or 128x128 blocks
    (square path) at random batch sizes."""
    n, nb, batch, relu = case
    say(f"[sweep] square {case}")
    seed = 9500 + n + batch
    q = n // nb
    w1 = S.draw(seed + 1, (nb, q, q), "normal", 1.0 / q, "bf16")
    w2 = S.draw(seed + 2, (nb, q, q), "normal", 1.0 / q, "bf16")
    x = S.draw(seed, (batch, n), "normal", 1.0, "bf16")
    dy = S.draw(seed + 3, (batch, n), "normal", 1.0, "bf16")
    act = 1 if relu else 0
    fac = O.dense_factors(w1, w2, n, n, sparse=n * n > (1 << 22))
    X, W1, W2 = dev(x, "bf16"), dev(w1, "bf16"), dev(w2, "bf16")
    y, z = api.monarch_forward(X, W1, W2, act)
    torch.cuda.synchronize()
    y_ref = O.forward(x, w1, w2, n, n, relu=relu, factors=fac)
    mask = dev(y_ref, "bf16") if relu else None
    dx, dw1, dw2 = api.monarch_backward(dev(dy, "bf16"), X, W1, W2, z, mask, act)
    torch.cuda.synchronize()
    rx, r1, r2 = O.backward(dy, x, w1, w2, n, n, relu=relu, y=y_ref, factors=fac)
    afac = O.dense_factors(np.abs(w1), np.abs(w2), n, n, sparse=n * n > (1 << 22))
    ys = O.forward(np.abs(x), np.abs(w1), np.abs(w2), n, n, factors=afac)
    sx, s1, s2 = O.backward(np.abs(dy), np.abs(x), np.abs(w1), np.abs(w2), n, n, relu=relu,
                            y=y_ref, factors=afac)
    errs = {"y": parity_error(host(y), y_ref, ys), "dx": parity_error(host(dx), rx, sx),
            "dw1": parity_error(host(dw1), r1, s1), "dw2": parity_error(host(dw2), r2, s2)}
    say(f"[sweep]   errors {errs}")
    for k, e in errs.items():
        assert e <= TOL["bf16"], (case, k, e)
