"""Pins of the DYAD-style oracle (CPU only): a literal loop over the index
maps, the A = 0 case against the separately pinned Monarch oracle, the exact
nonzero pattern, the parameter count, finite differences and
multilinearity."""
import numpy as np
import pytest

import oracle as O
from oracle import dyad as D

SHAPES = [(8, 8, 2), (12, 8, 4), (16, 24, 4), (9, 6, 3), (6, 6, 1), (6, 6, 6)]


def rand(rng, inp, out, nb, batch=4):
    s = D.dyad_sizes(inp, out, nb)
    shape = (nb, s["qo"], s["qi"])
    return rng.standard_normal(shape), rng.standard_normal(shape), rng.standard_normal((batch, inp))


def literal(x, wa, wb, inp, out):
    nb, qo, qi = wa.shape
    rows = []
    for xr in np.asarray(x, dtype=np.float64):
        y = [0.0] * out
        for r in range(nb):                      # contiguous blocks
            for k in range(qo):
                y[r * qo + k] += sum(wa[r, k, s] * xr[r * qi + s] for s in range(qi))
        for g in range(nb):                      # blocks on the residue-g features
            for p in range(qo):
                y[p * nb + g] += sum(wb[g, p, t] * xr[t * nb + g] for t in range(qi))
        rows.append(y)
    return np.array(rows)


@pytest.mark.parametrize("shape", SHAPES)
def test_literal_loop_matches(shape):
    rng = np.random.default_rng(1)
    wa, wb, x = rand(rng, *shape)
    assert np.allclose(D.forward(x, wa, wb, shape[0], shape[1]), literal(x, wa, wb, *shape[:2]),
                       atol=1e-12)


@pytest.mark.parametrize("n,nb", [(8, 2), (16, 4), (12, 3), (9, 3)])
def test_second_term_is_monarch_with_identity_first_factor(n, nb):
    """A = 0, square: Q_out·BD(B)·P_in is the Monarch matrix of R = identity
    blocks and L = B (b2 = nb)."""
    rng = np.random.default_rng(2)
    wa, wb, _ = rand(rng, n, n, nb)
    eye = np.broadcast_to(np.eye(n // nb), (nb, n // nb, n // nb)).copy()
    M = O.monarch_matrix(eye, wb, n, n)
    assert np.allclose(D.dyad_matrix(np.zeros_like(wa), wb, n, n), M, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
def test_nonzero_pattern(shape):
    """Entry (o, i) can be nonzero exactly when o and i sit in the same
    contiguous block or have the same residue mod nb."""
    inp, out, nb = shape
    rng = np.random.default_rng(3)
    wa, wb, _ = rand(rng, *shape)
    M = D.dyad_matrix(wa, wb, inp, out)
    qi, qo = inp // nb, out // nb
    o, i = np.meshgrid(np.arange(out), np.arange(inp), indexing="ij")
    allowed = (o // qo == i // qi) | (o % nb == i % nb)
    assert np.array_equal(M != 0, allowed)


def test_parameter_count():
    assert D.param_count(16384, 16384, 128) == 2 * 16384 * 16384 // 128
    assert D.param_count(768, 3072, 4) == 2 * 768 * 3072 // 4


@pytest.mark.parametrize("shape", SHAPES)
def test_finite_differences(shape):
    inp, out, nb = shape
    rng = np.random.default_rng(4)
    wa, wb, x = rand(rng, *shape, batch=3)
    dy = rng.standard_normal((3, out))
    dx, da, db = D.backward(dy, x, wa, wb, inp, out)

    def loss():
        return float(np.sum(dy * D.forward(x, wa, wb, inp, out)))
    h = 1e-6
    for arr, grad in ((x, dx), (wa, da), (wb, db)):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for idx in rng.choice(flat.size, size=min(10, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + h
            lp = loss()
            flat[idx] = old - h
            lm = loss()
            flat[idx] = old
            assert abs((lp - lm) / (2 * h) - gflat[idx]) <= 1e-6 * (1 + abs(gflat[idx]))


@pytest.mark.parametrize("shape", SHAPES)
def test_linearity_identities(shape):
    """Y = X·(BD(A) + Q·BD(B)·P)ᵀ: <dY, Y> = <dX, X> = <dA, A> + <dB, B>, and
    each term separately: <dA, A> = <dY, Y(A, 0)>, <dB, B> = <dY, Y(0, B)>."""
    inp, out, nb = shape
    rng = np.random.default_rng(5)
    wa, wb, x = rand(rng, *shape)
    dy = rng.standard_normal((x.shape[0], out))
    dx, da, db = D.backward(dy, x, wa, wb, inp, out)
    ref = np.sum(dy * D.forward(x, wa, wb, inp, out))
    assert abs(np.sum(dx * x) - ref) <= 1e-10 * (1 + abs(ref))
    ya = np.sum(dy * D.forward(x, wa, np.zeros_like(wb), inp, out))
    yb = np.sum(dy * D.forward(x, np.zeros_like(wa), wb, inp, out))
    assert abs(np.sum(da * wa) - ya) <= 1e-10 * (1 + abs(ya))
    assert abs(np.sum(db * wb) - yb) <= 1e-10 * (1 + abs(yb))


def test_bad_sizes_raise():
    with pytest.raises(ValueError):
        D.dyad_sizes(10, 8, 4)
