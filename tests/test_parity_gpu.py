"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: relative Frobenius error <= 1e-5 for fp32 and <= 2e-2 for bf16 inputs
with fp32 accumulation, per output tensor (Y; dX, dw1, dw2), and the same
bound for every row of each tensor (O.parity_error); bit-exact for 0/1
permutation blocks. Inputs come from the seeded generator module; no
oracle input or expected value comes from the GPU path.
"""
import sys

import numpy as np
import pytest

import oracle as O
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


def rand_layer(inp, out, b1, b2, batch, dtype, seed, x_dist="normal"):
    s = O.derive_sizes(inp, out, b1, b2)
    w1 = S.draw(seed + 1, (b1, s["q1o"], s["q1i"]), "normal", 1.0 / s["q1i"], dtype)
    w2 = S.draw(seed + 2, (b2, s["q2o"], s["q2i"]), "normal", 1.0 / s["q2i"], dtype)
    x = S.draw(seed, (batch, inp), x_dist, 1.0, dtype)
    dy = S.draw(seed + 3, (batch, out), "normal", 1.0, dtype)
    return x, w1, w2, dy


def factors_for(w1, w2, inp, out):
    """The oracle's factor matrices; sparse storage (same entries) when dense
    ones would be large."""
    return O.dense_factors(w1, w2, inp, out, sparse=inp * out > (1 << 22))


def check_layer(api, x, w1, w2, dy, inp, out, dtype, relu, with_bwd=True, label=""):
    """Forward (and backward) of one layer against the oracle. With ReLU the
    GPU backward takes the oracle's forward output as its mask source, so
    both sides mask the same entries."""
    say(f"[parity] {label} in={inp} out={out} b1={w1.shape[0]} b2={w2.shape[0]} "
        f"batch={x.shape[0]} {dtype} relu={relu}")
    act = 1 if relu else 0
    fac = factors_for(w1, w2, inp, out)
    X, W1, W2 = dev(x, dtype), dev(w1, dtype), dev(w2, dtype)
    y, z = api.monarch_forward(X, W1, W2, act)
    torch.cuda.synchronize()
    y_ref = O.forward(x, w1, w2, inp, out, relu=relu, factors=fac)
    # row scales: the same results from the absolute values of every input
    A = np.abs
    afac = factors_for(A(w1), A(w2), inp, out)
    ys = O.forward(A(x), A(w1), A(w2), inp, out, factors=afac)
    errs = {"y": O.parity_error(host(y), y_ref, ys)}
    if with_bwd:
        mask = dev(y_ref, dtype) if relu else None
        dx, dw1, dw2 = api.monarch_backward(dev(dy, dtype), X, W1, W2, z, mask, act)
        torch.cuda.synchronize()
        rx, r1, r2 = O.backward(dy, x, w1, w2, inp, out, relu=relu, y=y_ref, factors=fac)
        sx, s1, s2 = O.backward(A(dy), A(x), A(w1), A(w2), inp, out, relu=relu, y=y_ref,
                                factors=afac)
        errs.update(dx=O.parity_error(host(dx), rx, sx), dw1=O.parity_error(host(dw1), r1, s1),
                    dw2=O.parity_error(host(dw2), r2, s2))
    say(f"[parity]   errors {errs}")
    for k, e in errs.items():
        assert e <= TOL[dtype], (label, k, e)
    return errs


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def test_tiny_square_n16(api):
    w = S.WORKLOADS["tiny_square_n16_b4"]
    d = S.make_layer_inputs(w)
    check_layer(api, d["x"], d["w1"], d["w2"], d["dy"], 16, 16, "f32", False, label=w.name)


def test_square_n1024_b32(api):
    w = S.WORKLOADS["square_n1024_b32"]
    d = S.make_layer_inputs(w)
    check_layer(api, d["x"], d["w1"], d["w2"], d["dy"], 1024, 1024, "bf16", False, label=w.name)


def test_gpt2_ffn_up(api):
    w = S.WORKLOADS["gpt2_ffn_up_768x3072_nb4"]
    d = S.make_layer_inputs(w)
    check_layer(api, d["x"], d["w1"], d["w2"], d["dy"], 768, 3072, "bf16", False, label=w.name)


RECSYS = [n for n in S.WORKLOADS if n.startswith("recsys")]


@pytest.mark.parametrize("name", RECSYS)
def test_recsys_mlp_layers(api, name):
    """Each Monarch layer gated on its own at the fp32 bar. Layer 2 and the
    layer-1 backward take the oracle's hidden activation (rounded to fp32) as
    input, so both sides use the same ReLU mask."""
    w = S.WORKLOADS[name]
    l1, l2 = w.layers
    d1 = S.make_layer_inputs(w, 0, with_dy=True)
    d2 = S.make_layer_inputs(w, 1, with_dy=False)
    x, dy = d1["x"], d1["dy"]
    layers = [(d1["w1"], d1["w2"], l1.in_features, l1.out_features, True),
              (d2["w1"], d2["w2"], l2.in_features, l2.out_features, False)]
    y_ref, acts = O.mlp_forward(x, layers)
    h_ref = acts[1]
    dx_ref, grads = O.mlp_backward(dy, x, layers)
    # gradient reaching the hidden activation, from the oracle's layer-2 backward
    dh_ref, _, _ = O.backward(dy, h_ref, d2["w1"], d2["w2"], l2.in_features, l2.out_features)
    # row scales: each layer's results from the absolute values of its inputs
    A = np.abs
    a1, a2 = (A(d1["w1"]), A(d1["w2"])), (A(d2["w1"]), A(d2["w2"]))
    f1, f2 = (l1.in_features, l1.out_features), (l2.in_features, l2.out_features)
    sh = O.forward(A(x), *a1, *f1)
    sy = O.forward(A(h_ref), *a2, *f2)
    sdh, s21, s22 = O.backward(A(dy), A(h_ref), *a2, *f2)
    sx, s11, s12 = O.backward(A(dh_ref), A(x), *a1, *f1, relu=True, y=h_ref)
    say(f"[parity] {name}")
    X, H = dev(x, "f32"), dev(h_ref, "f32")
    A1 = (dev(d1["w1"], "f32"), dev(d1["w2"], "f32"))
    A2 = (dev(d2["w1"], "f32"), dev(d2["w2"], "f32"))
    h_gpu, z1 = api.monarch_forward(X, *A1, act=1)
    y_gpu, z2 = api.monarch_forward(H, *A2, act=0)
    dh, g21, g22 = api.monarch_backward(dev(dy, "f32"), H, *A2, z2, None, 0)
    dx, g11, g12 = api.monarch_backward(dev(dh_ref, "f32"), X, *A1, z1, H, 1)
    torch.cuda.synchronize()
    errs = dict(
        h=O.parity_error(host(h_gpu), h_ref, sh),
        y=O.parity_error(host(y_gpu), y_ref, sy),
        dh=O.parity_error(host(dh), dh_ref, sdh),
        dw1_l2=O.parity_error(host(g21), grads[1][0], s21),
        dw2_l2=O.parity_error(host(g22), grads[1][1], s22),
        dx=O.parity_error(host(dx), dx_ref, sx),
        dw1_l1=O.parity_error(host(g11), grads[0][0], s11),
        dw2_l1=O.parity_error(host(g12), grads[0][1], s12),
    )
    say(f"[parity]   errors {errs}")
    for k, e in errs.items():
        assert e <= TOL["f32"], (name, k, e)


def _mlp_chain_gpu(api, x, dy, d1, d2):
    """Both layers chained on the GPU (ReLU between): y and all gradients."""
    X = dev(x, "f32")
    A1 = (dev(d1["w1"], "f32"), dev(d1["w2"], "f32"))
    A2 = (dev(d2["w1"], "f32"), dev(d2["w2"], "f32"))
    h, z1 = api.monarch_forward(X, *A1, act=1)
    y, z2 = api.monarch_forward(h, *A2, act=0)
    dh, g21, g22 = api.monarch_backward(dev(dy, "f32"), h, *A2, z2, None, 0)
    dx, g11, g12 = api.monarch_backward(dh, X, *A1, z1, h, 1)
    torch.cuda.synchronize()
    return host(h), host(y), [host(t) for t in (dx, g11, g12, g21, g22)]


@pytest.mark.parametrize("name", ["recsys_mlp_10000x1024x512_nb4_b1000",
                                  "recsys_mlp_10000x1024x512_nb16_b10",
                                  "recsys_mlp_10000x1024x512_nb16_b1000"])
def test_recsys_mlp_end_to_end(api, name):
    """The two layers chained on the GPU. The forward is gated at the fp32
    bar (ReLU is continuous). A hidden entry whose ReLU mask differs between
    the two sides (a pre-activation within rounding of 0) changes its row's
    dX and every weight-gradient sum, so the backward is gated with the rows
    holding such entries excluded: the chain is run again on both sides over
    the remaining rows, whose masks must then all agree."""
    w = S.WORKLOADS[name]
    l1, l2 = w.layers
    d1 = S.make_layer_inputs(w, 0)
    d2 = S.make_layer_inputs(w, 1, with_dy=False)
    layers = [(d1["w1"], d1["w2"], l1.in_features, l1.out_features, True),
              (d2["w1"], d2["w2"], l2.in_features, l2.out_features, False)]
    x, dy = d1["x"], d1["dy"]
    y_ref, acts = O.mlp_forward(x, layers)
    # row scales: the chain from the absolute values of every input (all
    # hidden units active, which only enlarges the scale)
    alayers = [(np.abs(a), np.abs(b), fi, fo, r) for (a, b, fi, fo, r) in layers]
    h, y, grads_gpu = _mlp_chain_gpu(api, x, dy, d1, d2)
    assert O.parity_error(y, y_ref, O.mlp_forward(np.abs(x), alayers)[0]) <= TOL["f32"]
    flipped = ((h > 0) != (acts[1] > 0)).any(axis=1)
    say(f"[parity] {name}: rows with a differing relu mask entry: {int(flipped.sum())}")
    rows = np.flatnonzero(~flipped)
    assert rows.size >= 0.9 * x.shape[0]
    if flipped.any():
        x, dy = x[rows], dy[rows]
        _, acts = O.mlp_forward(x, layers)
        h, _, grads_gpu = _mlp_chain_gpu(api, x, dy, d1, d2)
        assert not ((h > 0) != (acts[1] > 0)).any()
    dx_ref, grads = O.mlp_backward(dy, x, layers)
    sdx, sg = O.mlp_backward(np.abs(dy), np.abs(x), alayers)
    refs = (dx_ref, grads[0][0], grads[0][1], grads[1][0], grads[1][1])
    scales = (sdx, sg[0][0], sg[0][1], sg[1][0], sg[1][1])
    for got, ref, sc in zip(grads_gpu, refs, scales):
        assert O.parity_error(got, ref, sc) <= TOL["f32"]


def test_square_n16384_full_size_sampled(api):
    """configs at full size (65536 x 16384, 128 blocks of 128x128, bf16), in
    the launch configuration the benchmark times. Sampled rows of Y and dX and
    sampled weight-gradient entries against the oracle (sparse storage of the
    same factor matrices); Euler identities on the whole tensors."""
    w = S.WORKLOADS["square_n16384_b128"]
    n, B = 16384, w.batch
    say("[parity] square_n16384 full size: drawing inputs")
    d = S.make_layer_inputs(w)
    X, W1, W2, DY = dev(d["x"], "bf16"), dev(d["w1"], "bf16"), dev(d["w2"], "bf16"), dev(d["dy"], "bf16")
    say("[parity] square_n16384: forward + backward on the GPU")
    y, z = api.monarch_forward(X, W1, W2)
    dx, dw1, dw2 = api.monarch_backward(DY, X, W1, W2, z)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 777, 4095, 30000, 65535])
    fac = O.dense_factors(d["w1"], d["w2"], n, n, sparse=True)
    say("[parity] square_n16384: oracle on sampled rows")
    y_ref = O.forward_rows(d["x"][rows], d["w1"], d["w2"], n, n, factors=fac)
    dx_ref = O.backward_dx_rows(d["dy"][rows], d["w1"], d["w2"], n, n, factors=fac)
    ey = O.rel_frobenius(host(y[torch.from_numpy(rows).cuda()]), y_ref)
    edx = O.rel_frobenius(host(dx[torch.from_numpy(rows).cuda()]), dx_ref)
    rks = [(0, 0, 0), (5, 17, 100), (127, 127, 127), (64, 3, 90)]
    gpt = [(0, 0, 0), (9, 100, 31), (127, 127, 127), (77, 12, 64)]
    say("[parity] square_n16384: oracle weight-gradient entries")
    er, el = O.weight_grad_entries(d["dy"], d["x"], d["w1"], d["w2"], n, n, rks, gpt, factors=fac)
    g1 = host(dw1)
    g2 = host(dw2)
    e1 = O.rel_frobenius(np.array([g1[i] for i in rks]), er)
    e2 = O.rel_frobenius(np.array([g2[i] for i in gpt]), el)
    say(f"[parity] square_n16384 sampled errors y={ey:.3e} dx={edx:.3e} dw1={e1:.3e} dw2={e2:.3e}")
    for e in (ey, edx, e1, e2):
        assert e <= TOL["bf16"]
    # Euler identities with dY = Y: <Y,Y> = <dX,X> = <dw1,w1> = <dw2,w2>
    dx2, dw1b, dw2b = api.monarch_backward(y, X, W1, W2, z)
    torch.cuda.synchronize()
    yy = torch.sum(y.double() * y.double()).item()
    vals = [torch.sum(dx2.double() * X.double()).item(),
            torch.sum(dw1b.double() * W1.double()).item(),
            torch.sum(dw2b.double() * W2.double()).item()]
    say(f"[parity] square_n16384 Euler: <Y,Y>={yy:.6e} others={vals}")
    for v in vals:
        assert abs(v - yy) <= 2e-2 * yy


def _dot64(a, b, chunk=8192):
    """<a, b> in fp64, accumulated over row chunks (bounded temporaries)."""
    tot = 0.0
    for i in range(0, a.shape[0], chunk):
        tot += torch.sum(a[i:i + chunk].double() * b[i:i + chunk].double()).item()
    return tot


def test_square_size_limit_ragged(api):
    """The fast path at its size limit: 131071 rows x 16384 (batch*out just
    under 2^31, the kernels' 32-bit offset bound) with a ragged tail of every
    tile size. Inputs are drawn on the device (seeded, the largest
    configuration's distributions); sampled rows of Y and dX, including the
    last ones, against the oracle; the weight gradients through the Euler
    identities (dY = Y), which hold at any size."""
    n, nb, B = 16384, 128, 131071
    assert B * n < 2 ** 31 and (B + 1) * n == 2 ** 31
    from monarch_block_diagonal_amd import binding as BD
    names = BD.monarch_describe(1, n, n, nb, nb, B, BD.BF16)
    assert all(k.startswith("sq128") or k == "reduce_dw" for k in names)
    say("[parity] size limit: drawing inputs on the device")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(S.seed_for(4, S.TID_X) + 7)
    X = torch.randn((B, n), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
    g.manual_seed(S.seed_for(4, S.TID_DY) + 7)
    DY = torch.randn((B, n), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
    w1 = S.draw(S.seed_for(4, S.TID_W1) + 7, (nb, 128, 128), "normal", 1.0 / 128, "bf16")
    w2 = S.draw(S.seed_for(4, S.TID_W2) + 7, (nb, 128, 128), "normal", 1.0 / 128, "bf16")
    W1, W2 = dev(w1, "bf16"), dev(w2, "bf16")
    say("[parity] size limit: forward + backward")
    y, z = api.monarch_forward(X, W1, W2)
    dx, _, _ = api.monarch_backward(DY, X, W1, W2, z)
    torch.cuda.synchronize()
    rows = np.array([0, 31, 65536, 131039, 131040, 131056, 131070])
    ridx = torch.from_numpy(rows).cuda()
    xr = host(X[ridx]).astype(np.float64)
    dyr = host(DY[ridx]).astype(np.float64)
    fac = O.dense_factors(w1, w2, n, n, sparse=True)
    say("[parity] size limit: oracle on sampled rows")
    ey = O.rel_frobenius(host(y[ridx]), O.forward_rows(xr, w1, w2, n, n, factors=fac))
    edx = O.rel_frobenius(host(dx[ridx]), O.backward_dx_rows(dyr, w1, w2, n, n, factors=fac))
    say(f"[parity] size limit sampled errors y={ey:.3e} dx={edx:.3e}")
    assert ey <= TOL["bf16"] and edx <= TOL["bf16"]
    del DY, dx
    dx2, dw1, dw2 = api.monarch_backward(y, X, W1, W2, z)
    torch.cuda.synchronize()
    yy = _dot64(y, y)
    vals = [_dot64(dx2, X), torch.sum(dw1.double() * W1.double()).item(),
            torch.sum(dw2.double() * W2.double()).item()]
    say(f"[parity] size limit Euler: <Y,Y>={yy:.6e} others={vals}")
    for v in vals:
        assert abs(v - yy) <= 2e-2 * yy


# --------------------------------------------------------------------------
# shapes: several tiles, ragged tails, rectangular, both dtypes, ReLU
# --------------------------------------------------------------------------

SHAPES = [
    # inp, out, b1, b2, batch
    (256, 256, 16, 16, 1000),
    (96, 160, 4, 8, 77),
    (160, 96, 8, 4, 130),
    (64, 64, 8, 8, 1),
    (512, 512, 4, 4, 333),
    (1024, 1024, 32, 32, 200),
    (2048, 2048, 16, 16, 129),
    (4096, 4096, 64, 64, 65),
    (16384, 16384, 128, 128, 96),
    # 128x128 blocks, 32, 64 or 128 of them: the bf16 fast path
    (4096, 4096, 32, 32, 1),
    (4096, 4096, 32, 32, 200),
    (8192, 8192, 64, 64, 77),
    (16384, 16384, 128, 128, 1000),
    (16384, 16384, 128, 128, 17),
    # 32x32 blocks, 8, 16 or 32 of them: the fused bf16 path
    (256, 256, 8, 8, 77),
    (512, 512, 16, 16, 130),
    (1024, 1024, 32, 32, 1),
    (1024, 1024, 32, 32, 4113),
    # 128x128 blocks, fewer blocks: generic path
    (1024, 1024, 8, 8, 77),
    (2048, 2048, 16, 16, 129),
    (768, 3072, 4, 4, 100),
    # bf16 256 x 256 tiles with ragged rows, ragged columns (520) and a K of
    # 300 (element-wise operand loads)
    (768, 3072, 4, 4, 1000),
    (600, 1040, 2, 2, 600),
    (1024, 2048, 2, 2, 513),
    # K = 520 (a last K tile of 8) on the 256 x 256 tile
    (1040, 1040, 2, 2, 600),
    # 256 x 192 tiles with ragged columns (170: element-wise loads, 176)
    (340, 680, 2, 2, 700),
    (352, 704, 2, 2, 700),
    (250, 100, 5, 2, 45),
    (36, 36, 6, 6, 17),
    (8, 8, 2, 4, 3),
    # bf16 stage-1 forward with weights held in registers: K = 256 with two
    # 256-column slices, K = 192 with one slice, one row, and K = 256 with a
    # column split of 32 (runs of n1 = q1o / b2 columns in stage 2's order)
    (1024, 2048, 4, 4, 333),
    (768, 1024, 4, 4, 17),
    (768, 3072, 4, 4, 1),
    (2048, 2048, 8, 8, 77),
    # the same kernel with a column split of 16, and with the stage-1 output
    # in its own order (q1o = 256 not a multiple of b2 = 512: no split)
    (1024, 1024, 4, 16, 100),
    (768, 1024, 4, 512, 33),
    # fp32 stage-1 forwards with K >= 512 and few 64 x 64 tiles (K split over
    # the eight waves of a workgroup): K = 512, and K = 525 with a tail and
    # rows starting off 16-byte boundaries
    (2048, 256, 4, 4, 300),
    (2100, 512, 4, 4, 100),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(api, shape, dtype):
    inp, out, b1, b2, batch = shape
    x, w1, w2, dy = rand_layer(inp, out, b1, b2, batch, dtype, seed=1000 + inp + out + batch)
    check_layer(api, x, w1, w2, dy, inp, out, dtype, relu=False, label="shape")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256, 16, 16, 300), (96, 160, 4, 8, 50),
                                   (16384, 16384, 128, 128, 64), (1024, 512, 16, 16, 100),
                                   (2048, 2048, 16, 16, 45), (4096, 4096, 32, 32, 45),
                                   (512, 512, 16, 16, 50), (1024, 1024, 32, 32, 129)],
                         ids=lambda s: "x".join(map(str, s)))
def test_shapes_relu(api, shape, dtype):
    inp, out, b1, b2, batch = shape
    x, w1, w2, dy = rand_layer(inp, out, b1, b2, batch, dtype, seed=7 + inp + batch)
    check_layer(api, x, w1, w2, dy, inp, out, dtype, relu=True, label="relu")


# --------------------------------------------------------------------------
# exact cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(16, 16, 4, 4, 8), (1024, 1024, 32, 32, 300),
                                   (16384, 16384, 128, 128, 64), (256, 256, 16, 16, 100),
                                   (4096, 4096, 32, 32, 33), (512, 512, 16, 16, 70),
                                   (48, 96, 2, 4, 10)], ids=lambda s: "x".join(map(str, s)))
def test_permutation_blocks_bit_exact(api, shape, dtype):
    """0/1 blocks (identity and cyclic shifts) make M a permutation matrix:
    the output must equal the permuted input bit for bit."""
    inp, out, b1, b2, batch = shape
    s = O.derive_sizes(inp, out, b1, b2)
    for a, c in ((0, 0), (1, 3)):
        sh1 = np.roll(np.eye(s["q1o"], s["q1i"]), a, axis=1).astype(np.float32)
        sh2 = np.roll(np.eye(s["q2o"], s["q2i"]), c, axis=1).astype(np.float32)
        w1 = np.stack([sh1] * b1)
        w2 = np.stack([sh2] * b2)
        x = S.draw(55 + a, (batch, inp), "normal", 1.0, dtype)
        # every row of M holds at most one 1, so the fp64 result is exact
        expect = O.forward(x, w1, w2, inp, out, factors=factors_for(w1, w2, inp, out))
        y, z = api.monarch_forward(dev(x, dtype), dev(w1, dtype), dev(w2, dtype))
        torch.cuda.synchronize()
        assert np.array_equal(host(y), expect), (shape, a, c)


def test_permutation_blocks_bit_exact_full_size(api):
    """The largest configuration's shape and launch (65536 x 16384, 128
    blocks of 128 x 128, bf16) with cyclic-shift 0/1 blocks, so M is a
    permutation matrix. Every row of Y and of dX must equal the permuted
    input bit for bit (the sign of a zero aside, see _report_mismatch). The permutation is read off the oracle's own sparse
    factor matrices (M = Qo·Ld·Pm·Rd, one 1 per row): Y[:, j] = X[:, pi(j)]
    and dX[:, pi(j)] = dY[:, j]."""
    n, nb, B = 16384, 128, 65536
    sh1 = np.roll(np.eye(128), 1, axis=1)
    sh2 = np.roll(np.eye(128), 3, axis=1)
    w1 = np.stack([sh1] * nb)
    w2 = np.stack([sh2] * nb)
    Rd, Pm, Ld, Qo = O.dense_factors(w1, w2, n, n, sparse=True)
    M = (Qo @ Ld @ Pm @ Rd).tocsr()
    M.eliminate_zeros()
    assert M.nnz == n and np.all(M.data == 1.0) and np.all(np.diff(M.indptr) == 1)
    pi = M.indices                      # row j of M has its 1 in column pi[j]
    assert np.array_equal(np.sort(pi), np.arange(n))
    say("[parity] permutation full size: drawing inputs")
    xb = S.bf16_bits(S.draw(4501, (B, n), "normal", 1.0, "bf16"))
    dyb = S.bf16_bits(S.draw(4502, (B, n), "normal", 1.0, "bf16"))
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)  # noqa: E731
    X, DY = to_dev(xb), to_dev(dyb)
    W1 = dev(w1.astype(np.float32), "bf16")
    W2 = dev(w2.astype(np.float32), "bf16")
    say("[parity] permutation full size: forward + backward")
    y, z = api.monarch_forward(X, W1, W2)
    dx, _, _ = api.monarch_backward(DY, X, W1, W2, z)
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    _report_mismatch("Y", yb, xb[:, pi])
    del yb
    dxb = dx.view(torch.int16).cpu().numpy().view(np.uint16)
    expect = np.empty_like(dyb)
    expect[:, pi] = dyb
    _report_mismatch("dX", dxb, expect)


def _report_mismatch(name, got, expect):
    """Bitwise comparison of bf16 patterns with the sign of zero made equal
    (0x8000 -> 0x0000 on both sides): the product sums a row's one 1·x term
    with 0·x terms from a +0 accumulator, and in IEEE arithmetic -0 + +0 is
    +0, so an input of -0.0 (the seeded normal draws hold exact zeros at
    about 2^-23 per value) comes out as +0.0, the same real number. On a
    mismatch, print where it is before failing."""
    got = np.where(got == 0x8000, np.uint16(0), got)
    expect = np.where(expect == 0x8000, np.uint16(0), expect)
    bad = got != expect
    n = int(bad.sum())
    if n:
        r, c = np.nonzero(bad)
        say(f"[parity] {name}: {n} entries differ in {np.unique(r).size} rows, "
            f"{np.unique(c).size} columns; rows {np.unique(r)[:12]} cols {np.unique(c)[:12]}")
        say(f"[parity] {name}: rows mod 16 {np.bincount(r % 16, minlength=16)}; "
            f"row blocks of 4096 {np.bincount(r // 4096)}; col blocks of 128 "
            f"{np.unique(c // 128)[:16]}")
        g32 = S.bf16_bits_to_f32(got[r[:8], c[:8]])
        e32 = S.bf16_bits_to_f32(expect[r[:8], c[:8]])
        say(f"[parity] {name}: first values got {g32} expected {e32}")
    assert n == 0, (name, n)


@pytest.mark.parametrize("shape", [(1024, 1024, 32, 32, 4096), (4096, 4096, 32, 32, 4100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_is_deterministic(api, shape):
    inp, out, b1, b2, batch = shape
    x, w1, w2, dy = rand_layer(inp, out, b1, b2, batch, "bf16", seed=99)
    X, W1, W2, DY = dev(x, "bf16"), dev(w1, "bf16"), dev(w2, "bf16"), dev(dy, "bf16")
    y, z = api.monarch_forward(X, W1, W2)
    a = api.monarch_backward(DY, X, W1, W2, z)
    b = api.monarch_backward(DY, X, W1, W2, z)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_batch_zero_backward_zeroes_weight_grads(api):
    from monarch_block_diagonal_amd import binding as B
    w1 = torch.randn(4, 4, 4, device="cuda:0")
    w2 = torch.randn(4, 4, 4, device="cuda:0")
    dw1 = torch.full_like(w1, 7.0)
    dw2 = torch.full_like(w2, 7.0)
    B.monarch_bwd(None, None, w1, w2, None, None, None, dw1, dw2, None, 0, 16, 16, 4, 4, 0,
                  B.F32, B.ACT_NONE)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw1).item() == 0 and torch.count_nonzero(dw2).item() == 0


def test_traced_events_time_each_kernel(api):
    from monarch_block_diagonal_amd import binding as B
    x, w1, w2, dy = rand_layer(1024, 1024, 32, 32, 4096, "bf16", seed=5)
    X, W1, W2 = dev(x, "bf16"), dev(w1, "bf16"), dev(w2, "bf16")
    names = B.monarch_describe(0, 1024, 1024, 32, 32, 4096, B.BF16)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    y = torch.empty(4096, 1024, dtype=torch.bfloat16, device="cuda:0")
    z = torch.empty_like(y)
    B.monarch_fwd(X, W1, W2, y, z, 1024, 1024, 32, 32, 4096, B.BF16, B.ACT_NONE, events=ev)
    torch.cuda.synchronize()
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(names))]
    assert all(t >= 0 for t in times)
    y_ref = O.forward(x, w1, w2, 1024, 1024)
    assert O.rel_frobenius(host(y), y_ref) <= TOL["bf16"]


def test_autograd_function(api):
    x, w1, w2, dy = rand_layer(256, 256, 16, 16, 64, "f32", seed=3)
    X = dev(x, "f32").requires_grad_()
    W1 = dev(w1, "f32").requires_grad_()
    W2 = dev(w2, "f32").requires_grad_()
    y = api.MonarchLinearFunction.apply(X, W1, W2, 1)
    y.backward(dev(dy, "f32"))
    y_ref = O.forward(x, w1, w2, 256, 256, relu=True)
    rx, r1, r2 = O.backward(dy, x, w1, w2, 256, 256, relu=True, y=y_ref)
    assert O.rel_frobenius(host(y), y_ref) <= 1e-5
    for got, ref in ((X.grad, rx), (W1.grad, r1), (W2.grad, r2)):
        assert O.rel_frobenius(host(got), ref) <= 1e-5
