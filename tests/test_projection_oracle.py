"""Pins of the projection oracle against facts the pages and mathematics fix
(CPU only). The oracle's own SVD is never re-called as a reference: every
check goes through the Monarch product (monarch_oracle.monarch_matrix), the
page's rearrangement, or a comparison against other candidate factors."""
import numpy as np
import pytest

import oracle as O
from oracle import monarch_projection as PJ

# Definition C.3 shapes: out = b1 * b2 (square with b = sqrt(n), and rectangular)
SHAPES = [(16, 16, 4, 4), (12, 8, 2, 4), (32, 32, 8, 4), (32, 32, 4, 8), (64, 64, 8, 8),
          (20, 6, 2, 3)]


def rand_factors(rng, inp, out, b1, b2):
    s = O.derive_sizes(inp, out, b1, b2)
    w1 = rng.standard_normal((b1, s["q1o"], s["q1i"]))
    w2 = rng.standard_normal((b2, s["q2o"], s["q2i"]))
    return w1, w2


@pytest.mark.parametrize("shape", SHAPES)
def test_projection_reproduces_monarch_inputs(shape):
    """A Monarch matrix is its own projection (the fit is exact)."""
    inp, out, b1, b2 = shape
    rng = np.random.default_rng(11)
    w1, w2 = rand_factors(rng, inp, out, b1, b2)
    m = O.monarch_matrix(w1, w2, inp, out)
    p1, p2 = PJ.project(m, inp, out, b1, b2)
    assert O.rel_frobenius(O.monarch_matrix(p1, p2, inp, out), m) < 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_projection_is_optimal_against_other_factors(shape):
    """No perturbed or random Monarch factor pair comes closer to M."""
    inp, out, b1, b2 = shape
    rng = np.random.default_rng(12)
    m = rng.standard_normal((out, inp))
    p1, p2 = PJ.project(m, inp, out, b1, b2)
    best = np.linalg.norm(m - O.monarch_matrix(p1, p2, inp, out))
    for eps in (1e-4, 1e-2, 0.3, 3.0):
        for _ in range(8):
            q1 = p1 + eps * rng.standard_normal(p1.shape)
            q2 = p2 + eps * rng.standard_normal(p2.shape)
            assert np.linalg.norm(m - O.monarch_matrix(q1, q2, inp, out)) >= best * (1 - 1e-12)
    for _ in range(8):
        q1, q2 = rand_factors(rng, inp, out, b1, b2)
        assert np.linalg.norm(m - O.monarch_matrix(q1, q2, inp, out)) >= best


@pytest.mark.parametrize("shape", SHAPES)
def test_projection_is_idempotent(shape):
    inp, out, b1, b2 = shape
    rng = np.random.default_rng(13)
    m = rng.standard_normal((out, inp))
    p1, p2 = PJ.project(m, inp, out, b1, b2)
    mh = O.monarch_matrix(p1, p2, inp, out)
    r1, r2 = PJ.project(mh, inp, out, b1, b2)
    assert O.rel_frobenius(O.monarch_matrix(r1, r2, inp, out), mh) < 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_projected_slices_are_rank_one_and_residual_orthogonal(shape):
    """In the page's rearrangement every slice of the fit has rank one, and
    the residual is orthogonal to the fit slice by slice (a wrong scaling of
    sigma breaks this)."""
    inp, out, b1, b2 = shape
    rng = np.random.default_rng(14)
    m = rng.standard_normal((out, inp))
    p1, p2 = PJ.project(m, inp, out, b1, b2)
    mh = O.monarch_matrix(p1, p2, inp, out)
    fit = PJ.slices(mh, inp, out, b1, b2)
    res = PJ.slices(m - mh, inp, out, b1, b2)
    for g in range(b2):
        for r in range(b1):
            sv = np.linalg.svd(fit[g, r], compute_uv=False)
            if len(sv) > 1:
                assert sv[1] <= 1e-12 * sv[0]
            assert abs(np.sum(fit[g, r] * res[g, r])) <= 1e-10 * np.sum(fit[g, r] ** 2)


def test_slice_view_matches_the_closed_form():
    """slices[g, r] of a Monarch matrix is the outer product L[g, :, r] R[r, g, :]
    (Definition C.3 entries), written out as loops."""
    inp, out, b1, b2 = 12, 8, 2, 4
    rng = np.random.default_rng(15)
    w1, w2 = rand_factors(rng, inp, out, b1, b2)
    sl = PJ.slices(O.monarch_matrix(w1, w2, inp, out), inp, out, b1, b2)
    for g in range(b2):
        for r in range(b1):
            for p in range(out // b2):
                for s in range(inp // b1):
                    assert abs(sl[g, r, p, s] - w2[g, p, r] * w1[r, g, s]) < 1e-12


def test_sign_convention():
    rng = np.random.default_rng(16)
    m = rng.standard_normal((16, 16))
    p1, _ = PJ.project(m, 16, 16, 4, 4)
    for r in range(4):
        for g in range(4):
            v = p1[r, g]
            assert v[int(np.argmax(np.abs(v)))] > 0


def test_not_applicable_shapes_raise():
    for shape in [(16, 16, 2, 4), (768, 3072, 4, 4), (15, 8, 2, 4)]:
        assert not PJ.projection_applies(*shape)
        with pytest.raises(ValueError):
            PJ.project(np.zeros((shape[1], shape[0])), *shape)


def test_planted_transposed_slice_is_caught():
    """Fitting the transposed slice (roles of p and s swapped) is not optimal."""
    inp, out, b1, b2 = 16, 16, 4, 4
    rng = np.random.default_rng(17)
    m = rng.standard_normal((out, inp))
    p1, p2 = PJ.project(m, inp, out, b1, b2)
    best = np.linalg.norm(m - O.monarch_matrix(p1, p2, inp, out))
    # wrong: swap the factor roles within each slice
    w1 = np.transpose(p2, (2, 0, 1)).copy()       # R[r, g, :] <- L[g, :, r]
    w2 = np.transpose(p1, (1, 2, 0)).copy()       # L[g, :, r] <- R[r, g, :]
    assert np.linalg.norm(m - O.monarch_matrix(w1, w2, inp, out)) > best * 1.01
