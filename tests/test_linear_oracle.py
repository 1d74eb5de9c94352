"""Pins of the MonarchLinear-variant oracle (explicit mid, zero-padded input,
truncated output, bias) against facts the pages and mathematics fix (CPU
only). Every check goes through something other than the dense factor chain
it tests: the page's printed parameter shapes, the separately pinned
monarch_oracle, a literal loop over the index maps, invariants of padding and
truncation, finite differences, or the multilinearity identities."""
import numpy as np
import pytest

import oracle as O
from oracle import monarch_linear as ML

# (in, out, mid, nb1, nb2): expanding (mid = in_ext), contracting, padded
# in/out, mid != out (Qo != Pmᵀ), unequal block counts
GEN_SHAPES = [
    (8, 16, 8, 2, 2),        # expanding, mid = in
    (16, 8, 8, 2, 2),        # contracting, mid = out
    (10, 7, 8, 4, 4),        # both padded (page rule, else branch)
    (5, 13, 8, 4, 4),        # expanding with padding (page rule: mid = in_ext)
    (12, 20, 12, 3, 2),      # mid = in, unequal block counts
    (9, 6, 12, 4, 3),        # padded in, mid > out
]


def rand_layer(rng, inp, out, mid, b1, b2, batch=5):
    s = ML.general_sizes(inp, out, mid, b1, b2)
    w1 = rng.standard_normal((b1, s["q1o"], s["q1i"]))
    w2 = rng.standard_normal((b2, s["q2o"], s["q2i"]))
    x = rng.standard_normal((batch, inp))
    bias = rng.standard_normal(out)
    return s, w1, w2, x, bias


def literal_forward(x, w1, w2, inp, out, mid, bias=None, relu=False):
    """Pure-Python loop over the index maps: zero-pad x to whole blocks, stage
    1 per block, the stride gather, stage 2 per block, the inverse scatter,
    keep the first `out` features."""
    b1, q1o, q1i = w1.shape
    b2, q2o, q2i = w2.shape
    rows = []
    for xr in np.asarray(x, dtype=np.float64):
        xe = [0.0] * (b1 * q1i)
        for i in range(inp):
            xe[i] = float(xr[i])
        z = [0.0] * mid
        for r in range(b1):
            for k in range(q1o):
                z[r * q1o + k] = sum(w1[r, k, s] * xe[r * q1i + s] for s in range(q1i))
        w = [0.0] * mid
        for g in range(b2):
            for t in range(q2i):
                w[g * q2i + t] = z[t * b2 + g]
        v = [0.0] * (b2 * q2o)
        for g in range(b2):
            for p in range(q2o):
                v[g * q2o + p] = sum(w2[g, p, t] * w[g * q2i + t] for t in range(q2i))
        ye = [0.0] * (b2 * q2o)
        for g in range(b2):
            for p in range(q2o):
                ye[p * b2 + g] = v[g * q2o + p]
        yr = ye[:out]
        if bias is not None:
            yr = [a + float(b) for a, b in zip(yr, bias)]
        if relu:
            yr = [max(a, 0.0) for a in yr]
        rows.append(yr)
    return np.array(rows)


def test_page_parameter_shapes():
    """blkdiag shapes of the MonarchLinear constructor for hand-worked sizes."""
    cases = {
        # (in, out, nb): (w1 shape, w2 shape, mid)
        (768, 3072, 4): ((4, 192, 192), (4, 768, 192), 768),     # expanding branch
        (3072, 768, 4): ((4, 192, 768), (4, 192, 192), 768),     # else branch
        (1024, 1024, 4): ((4, 256, 256), (4, 256, 256), 1024),
        (10, 7, 4): ((4, 2, 3), (4, 2, 2), 8),                   # ceil: 3 and 2; 12 >= 8
        (5, 13, 4): ((4, 2, 2), (4, 4, 2), 8),                   # ceil: 2 and 4; 8 < 16
        (10000, 1024, 16): ((16, 64, 625), (16, 64, 64), 1024),
    }
    for (i, o, nb), (s1, s2, mid) in cases.items():
        s = ML.linear_sizes(i, o, nb)
        assert (s["b1"], s["q1o"], s["q1i"]) == s1
        assert (s["b2"], s["q2o"], s["q2i"]) == s2
        assert s["mid"] == mid


@pytest.mark.parametrize("shape", [(16, 16, 4, 4), (12, 8, 2, 4), (768 // 32, 3072 // 32, 4, 4)])
def test_reduces_to_the_pinned_oracle(shape):
    """Divisible sizes, mid = out, no bias: the same numbers as monarch_oracle."""
    inp, out, b1, b2 = shape
    rng = np.random.default_rng(1)
    s, w1, w2, x, _ = rand_layer(rng, inp, out, out, b1, b2)
    dy = rng.standard_normal((x.shape[0], out))
    y = ML.forward_ex(x, w1, w2, inp, out, out)
    assert np.allclose(y, O.forward(x, w1, w2, inp, out), rtol=1e-13, atol=1e-13)
    dx, dw1, dw2, _ = ML.backward_ex(dy, x, w1, w2, inp, out, out)
    rx, r1, r2 = O.backward(dy, x, w1, w2, inp, out)
    for a, b in ((dx, rx), (dw1, r1), (dw2, r2)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", GEN_SHAPES)
@pytest.mark.parametrize("relu", [False, True])
def test_literal_loop_matches(shape, relu):
    rng = np.random.default_rng(2)
    s, w1, w2, x, bias = rand_layer(rng, *shape)
    inp, out, mid = shape[:3]
    y = ML.forward_ex(x, w1, w2, inp, out, mid, bias, relu)
    assert np.allclose(y, literal_forward(x, w1, w2, inp, out, mid, bias, relu), atol=1e-12)


@pytest.mark.parametrize("shape", GEN_SHAPES)
def test_padding_columns_are_zero_inputs(shape):
    """Weights on the padded input positions change nothing and receive zero
    gradient; padding the input by hand gives the same output."""
    inp, out, mid, b1, b2 = shape
    rng = np.random.default_rng(3)
    s, w1, w2, x, bias = rand_layer(rng, *shape)
    y = ML.forward_ex(x, w1, w2, inp, out, mid, bias)
    pad = s["in_ext"] - inp
    if pad:
        padded = [(f // s["q1i"], f % s["q1i"]) for f in range(inp, s["in_ext"])]
        w1b = w1.copy()
        for r, c in padded:
            w1b[r, :, c] = rng.standard_normal(s["q1o"])
        assert np.allclose(ML.forward_ex(x, w1b, w2, inp, out, mid, bias), y, atol=1e-12)
        dy = rng.standard_normal(y.shape)
        _, dw1, _, _ = ML.backward_ex(dy, x, w1, w2, inp, out, mid, bias)
        for r, c in padded:
            assert np.all(dw1[r, :, c] == 0.0)
    xe = np.concatenate([x, np.zeros((x.shape[0], pad))], axis=1)
    assert np.allclose(ML.forward_ex(xe, w1, w2, s["in_ext"], out, mid, bias), y, atol=1e-12)


@pytest.mark.parametrize("shape", GEN_SHAPES)
def test_truncation_keeps_the_first_features(shape):
    inp, out, mid, b1, b2 = shape
    rng = np.random.default_rng(4)
    s, w1, w2, x, _ = rand_layer(rng, *shape)
    full = ML.forward_ex(x, w1, w2, inp, s["out_ext"], mid)
    assert np.allclose(ML.forward_ex(x, w1, w2, inp, out, mid), full[:, :out], atol=1e-12)


def test_output_scatter_has_its_own_size():
    """mid != out: the output scatter is a permutation of out_ext features, not
    Pmᵀ (mid features); leaving it out (stage 2's block-major order kept)
    gives a different layer, and the literal loop sides with the oracle."""
    inp, out, mid, b1, b2 = 8, 16, 8, 2, 2
    rng = np.random.default_rng(5)
    s, w1, w2, x, _ = rand_layer(rng, inp, out, mid, b1, b2)
    E, Rd, Pm, Ld, Qo, T = ML.dense_factors_ex(w1, w2, inp, out, mid)
    assert Qo.shape == (16, 16) and Pm.shape == (8, 8)
    lit = literal_forward(x, w1, w2, inp, out, mid)
    wrong = x @ (T @ Ld @ Pm @ Rd @ E).T          # planted mistake: no output scatter
    assert not np.allclose(wrong, lit)
    assert np.allclose(ML.forward_ex(x, w1, w2, inp, out, mid), lit, atol=1e-12)


@pytest.mark.parametrize("shape", GEN_SHAPES)
def test_bias_is_added_before_the_activation(shape):
    inp, out, mid, b1, b2 = shape
    rng = np.random.default_rng(6)
    s, w1, w2, x, bias = rand_layer(rng, *shape)
    y0 = ML.forward_ex(x, w1, w2, inp, out, mid)
    yb = ML.forward_ex(x, w1, w2, inp, out, mid, bias)
    assert np.allclose(yb - y0, np.broadcast_to(bias, y0.shape), atol=1e-12)
    yr = ML.forward_ex(x, w1, w2, inp, out, mid, bias, relu=True)
    assert np.array_equal(yr, np.maximum(yb, 0.0))


@pytest.mark.parametrize("shape", GEN_SHAPES)
@pytest.mark.parametrize("relu", [False, True])
def test_finite_differences(shape, relu):
    inp, out, mid, b1, b2 = shape
    rng = np.random.default_rng(7)
    s, w1, w2, x, bias = rand_layer(rng, *shape, batch=3)
    dy = rng.standard_normal((3, out))

    def loss(x_, w1_, w2_, b_):
        return float(np.sum(dy * ML.forward_ex(x_, w1_, w2_, inp, out, mid, b_, relu)))

    dx, dw1, dw2, db = ML.backward_ex(dy, x, w1, w2, inp, out, mid, bias, relu)
    h = 1e-6
    for name, arr, grad in (("x", x, dx), ("w1", w1, dw1), ("w2", w2, dw2), ("b", bias, db)):
        flat = arr.reshape(-1)
        for idx in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + h
            lp = loss(x, w1, w2, bias)
            flat[idx] = old - h
            lm = loss(x, w1, w2, bias)
            flat[idx] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - grad.reshape(-1)[idx]) <= 1e-5 * (1 + abs(num)), (name, idx)


@pytest.mark.parametrize("shape", GEN_SHAPES)
def test_multilinearity_identities(shape):
    """Y - bias is linear in each of X, w1, w2 separately: <dY, Y - b> equals
    <dX, X>, <dw1, w1> and <dw2, w2>; and <dY, b> = <dbias, b>."""
    inp, out, mid, b1, b2 = shape
    rng = np.random.default_rng(8)
    s, w1, w2, x, bias = rand_layer(rng, *shape)
    dy = rng.standard_normal((x.shape[0], out))
    y = ML.forward_ex(x, w1, w2, inp, out, mid, bias)
    dx, dw1, dw2, db = ML.backward_ex(dy, x, w1, w2, inp, out, mid, bias)
    ref = np.sum(dy * (y - bias))
    for a, b in ((dx, x), (dw1, w1), (dw2, w2)):
        assert abs(np.sum(a * b) - ref) <= 1e-10 * (1 + abs(ref))
    assert abs(np.sum(dy * bias) - np.sum(db * bias)) <= 1e-10 * (1 + abs(np.sum(dy * bias)))


def test_invalid_sizes_raise():
    with pytest.raises(ValueError):
        ML.general_sizes(8, 8, 10, 4, 4)      # mid not divisible by the block counts
    with pytest.raises(ValueError):
        ML.general_sizes(0, 8, 8, 2, 2)
