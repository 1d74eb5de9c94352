"""Pins of the k-factor (hypercube) oracle against facts the page and the
mathematics fix (CPU only): the page's matrix counts, the k = 2 case against
the separately pinned two-factor oracle, a literal loop over multi-indices,
identity and permutation blocks, finite differences and multilinearity."""
import itertools

import numpy as np
import pytest

import oracle as O
from oracle import monarch_hypercube as H

DIMS = [(2, 3), (3, 2, 4), (2, 3, 2, 2), (4, 4), (5,)]


def rand_ws(rng, dims):
    return [rng.standard_normal(s) for s in H.weight_shapes(dims)]


def test_page_lattice_counts():
    """12288 units as 16 x 24 x 32: 768 matrices of 16 x 16, 512 of 24 x 24 and
    384 of 32 x 32 (the page's third round lists 16 x 16, but its last axis is
    32 long)."""
    shapes = H.weight_shapes((16, 24, 32))
    assert shapes == [(768, 16, 16), (512, 24, 24), (384, 32, 32)]
    assert H.param_count((16, 24, 32)) == 12288 * (16 + 24 + 32)


@pytest.mark.parametrize("ab", [(2, 3), (4, 4), (3, 5), (4, 2)])
def test_two_axes_is_the_transposed_two_factor_monarch(ab):
    """k = 2 on the lattice [A, B]: round 1 (axis 0, B matrices of A x A) then
    round 2 (axis 1, A matrices of B x B) equals Tᵀ·M·T with M the two-factor
    Monarch matrix of R = round-1 weights (b1 = B blocks) and L = round-2
    weights (b2 = A blocks), and T the lattice transpose (stride permutation)."""
    A, B = ab
    rng = np.random.default_rng(1)
    w1, w2 = rand_ws(rng, (A, B))
    n = A * B
    M = O.monarch_matrix(w1, w2, n, n)
    T = O.stride_permutation(n, B)
    assert np.allclose(H.hyper_matrix([w1, w2], (A, B)), T.T @ M @ T, atol=1e-12)


def literal(x, ws, dims):
    """Pure-Python loop: for every round, every fiber and every output
    position, sum over the input positions along that axis."""
    k = len(dims)
    rows = []
    for xr in np.asarray(x, dtype=np.float64):
        cur = {idx: float(xr[np.ravel_multi_index(idx, dims)])
               for idx in itertools.product(*[range(d) for d in dims])}
        for j in range(k):
            others = [d for i, d in enumerate(dims) if i != j]
            nxt = {}
            for idx in cur:
                o_idx = tuple(v for i, v in enumerate(idx) if i != j)
                f = int(np.ravel_multi_index(o_idx, others)) if others else 0
                o = idx[j]
                s = 0.0
                for a in range(dims[j]):
                    src = idx[:j] + (a,) + idx[j + 1:]
                    s += ws[j][f][o, a] * cur[src]
                nxt[idx] = s
            cur = nxt
        rows.append([cur[np.unravel_index(u, dims)] for u in range(int(np.prod(dims)))])
    return np.array(rows)


@pytest.mark.parametrize("dims", DIMS)
def test_literal_loop_matches(dims):
    rng = np.random.default_rng(2)
    ws = rand_ws(rng, dims)
    x = rng.standard_normal((3, int(np.prod(dims))))
    assert np.allclose(H.forward(x, ws, dims), literal(x, ws, dims), atol=1e-12)


@pytest.mark.parametrize("dims", DIMS)
def test_identity_and_shift_blocks(dims):
    n = int(np.prod(dims))
    eye = [np.broadcast_to(np.eye(d), s).copy() for d, s in zip(dims, H.weight_shapes(dims))]
    assert np.array_equal(H.hyper_matrix(eye, dims), np.eye(n))
    # cyclic shifts along every axis: the layer is a permutation of the units
    shift = [np.broadcast_to(np.roll(np.eye(d), 1, axis=0), s).copy()
             for d, s in zip(dims, H.weight_shapes(dims))]
    M = H.hyper_matrix(shift, dims)
    assert np.array_equal(M.sum(axis=0), np.ones(n)) and np.array_equal(M.sum(axis=1), np.ones(n))
    idx = np.arange(n).reshape(dims)
    expect = idx.copy()
    for j in range(len(dims)):
        expect = np.roll(expect, 1, axis=j)
    # unit u of the output takes the input unit shifted back by one on every axis
    assert np.array_equal(M @ np.arange(n, dtype=float), expect.reshape(-1).astype(float))


@pytest.mark.parametrize("dims", DIMS)
def test_each_round_moves_along_its_axis_only(dims):
    rng = np.random.default_rng(3)
    ws = rand_ws(rng, dims)
    n = int(np.prod(dims))
    for j, w in enumerate(ws):
        F = H.round_matrix(w, dims, j)
        for u in range(n):
            nz = np.nonzero(F[:, u])[0]
            iu = np.unravel_index(u, dims)
            for v in nz:
                iv = np.unravel_index(v, dims)
                assert all(a == b for i, (a, b) in enumerate(zip(iu, iv)) if i != j)


@pytest.mark.parametrize("dims", DIMS)
def test_finite_differences(dims):
    rng = np.random.default_rng(4)
    ws = rand_ws(rng, dims)
    n = int(np.prod(dims))
    x = rng.standard_normal((2, n))
    dy = rng.standard_normal((2, n))
    dx, dws = H.backward(dy, x, ws, dims)

    def loss():
        return float(np.sum(dy * H.forward(x, ws, dims)))
    h = 1e-6
    for arr, grad in [(x, dx)] + list(zip(ws, dws)):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for idx in rng.choice(flat.size, size=min(10, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + h
            lp = loss()
            flat[idx] = old - h
            lm = loss()
            flat[idx] = old
            assert abs((lp - lm) / (2 * h) - gflat[idx]) <= 1e-6 * (1 + abs(gflat[idx]))


@pytest.mark.parametrize("dims", DIMS)
def test_multilinearity_identities(dims):
    """Y is linear in X and in every round's weights: <dY, Y> = <dX, X> = <dw_j, w_j>."""
    rng = np.random.default_rng(5)
    ws = rand_ws(rng, dims)
    n = int(np.prod(dims))
    x = rng.standard_normal((4, n))
    dy = rng.standard_normal((4, n))
    y = H.forward(x, ws, dims)
    dx, dws = H.backward(dy, x, ws, dims)
    ref = np.sum(dy * y)
    assert abs(np.sum(dx * x) - ref) <= 1e-10 * (1 + abs(ref))
    for w, dw in zip(ws, dws):
        assert abs(np.sum(dw * w) - ref) <= 1e-10 * (1 + abs(ref))


def test_round_order_matters():
    """A planted mistake (rounds in reverse axis order) gives another layer."""
    rng = np.random.default_rng(6)
    dims = (2, 3, 4)
    ws = rand_ws(rng, dims)
    M = H.hyper_matrix(ws, dims)
    Fs = [H.round_matrix(w, dims, j) for j, w in enumerate(ws)]
    assert not np.allclose(M, Fs[0] @ Fs[1] @ Fs[2])


@pytest.mark.parametrize("dims", DIMS)
def test_fiber_form_matches_the_dense_form(dims):
    rng = np.random.default_rng(7)
    ws = rand_ws(rng, dims)
    n = int(np.prod(dims))
    x = rng.standard_normal((3, n))
    dy = rng.standard_normal((3, n))
    assert np.allclose(H.forward_fibers(x, ws, dims), H.forward(x, ws, dims), atol=1e-12)
    gx, gws = H.backward_fibers(dy, x, ws, dims)
    rx, rws = H.backward(dy, x, ws, dims)
    assert np.allclose(gx, rx, atol=1e-12)
    for a, b in zip(gws, rws):
        assert np.allclose(a, b, atol=1e-12)
