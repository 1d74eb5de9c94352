"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each check is chosen so that a plausible slip in the oracle (a transposed
permutation, a dropped output permutation, a transposed block, factors in the
wrong order, a missing term in the backward pass) fails at least one of them;
the planted-mistake tests at the end show that for the main slips.
"""
import os

import numpy as np
import pytest

import oracle as O
from monarch_block_diagonal_amd import synthetic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rand_factors(inp, out, b1, b2, seed=0):
    s = O.derive_sizes(inp, out, b1, b2)
    r = _rng(seed)
    w1 = r.standard_normal((b1, s["q1o"], s["q1i"]))
    w2 = r.standard_normal((b2, s["q2o"], s["q2i"]))
    return w1, w2


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                lhs, rhs = line.split(":")
                rows.append((lhs.split(), rhs.strip()))
    return rows


# --------------------------------------------------------------------------
# P1: the 4-unit permutation printed on the page
# --------------------------------------------------------------------------

def check_stride_permutation_fixture():
    for lhs, rhs in _read_golden("stride_permutation_4units.txt"):
        n, nb = int(lhs[0]), int(lhs[1])
        order = [int(v) for v in rhs.split()]
        x = np.arange(n, dtype=np.float64) + 10.0
        got = O.stride_permutation(n, nb) @ x
        assert np.array_equal(got, x[order])


def test_stride_permutation_page_example():
    check_stride_permutation_fixture()


def test_stride_permutation_is_reshape_transpose():
    # "reshape (q2i, nb2) then transpose": numpy's own reshape/transpose
    for mid, nb2 in [(8, 2), (12, 3), (16, 4), (24, 8), (6, 6), (7, 1)]:
        x = np.arange(mid, dtype=np.float64)
        got = O.stride_permutation(mid, nb2) @ x
        assert np.array_equal(got, x.reshape(mid // nb2, nb2).T.ravel())
        q = O.output_permutation(mid, nb2)
        # with mid = out the output permutation undoes P
        assert np.array_equal(q @ got, x)


# --------------------------------------------------------------------------
# lattice view of the square case (rows by one factor, columns by the other)
# --------------------------------------------------------------------------

def _groups_of(M):
    """Connected groups of input indices that M mixes together (M's pattern)."""
    n = M.shape[1]
    groups = []
    seen = set()
    for i in range(n):
        if i in seen:
            continue
        rows = np.nonzero(M[:, i])[0]
        cols = sorted(set(np.nonzero(M[rows, :])[1].tolist()))
        groups.append(cols)
        seen.update(cols)
    return sorted(groups)


def test_lattice_groups_page_example():
    fix = dict((lhs[0], [sorted(int(v) for v in g.split()) for g in rhs.split("|")])
               for lhs, rhs in _read_golden("lattice_groups_4units.txt"))
    w1, w2 = _rand_factors(4, 4, 2, 2, seed=1)
    eye = np.stack([np.eye(2)] * 2)
    # R alone (L = identity blocks) mixes the lattice rows; L alone the columns
    assert _groups_of(O.monarch_matrix(w1, eye, 4, 4)) == sorted(fix["rows"])
    assert _groups_of(O.monarch_matrix(eye, w2, 4, 4)) == sorted(fix["columns"])


@pytest.mark.parametrize("b1,b2", [(4, 4), (2, 8), (8, 2), (8, 8), (4, 16)])
def test_lattice_view_square_and_rectangular(b1, b2):
    # Definition C.3 case (b1*b2 = n): x viewed as a (b1, n/b1) lattice; R
    # transforms each lattice row, L each lattice column, output read back in
    # lattice order. Written with einsum, independent of the dense factors.
    n = b1 * b2
    w1, w2 = _rand_factors(n, n, b1, b2, seed=2)
    X = _rng(3).standard_normal((5, n))
    Xm = X.reshape(5, b1, n // b1)
    Z = np.einsum("rks,brs->brk", w1, Xm)              # (B, b1 rows, b2 cols)
    Y = np.einsum("gpt,btg->bpg", w2, Z).reshape(5, n)
    np.testing.assert_allclose(O.forward(X, w1, w2, n, n), Y, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P2: closed form and rank-1 slices in the Definition C.3 case
# --------------------------------------------------------------------------

def check_closed_form(n, b1, b2, seed=4):
    w1, w2 = _rand_factors(n, n, b1, b2, seed=seed)
    M = O.monarch_matrix(w1, w2, n, n)
    q1i = n // b1
    # hand derivation: M[p*b2 + g, r*q1i + s] = L[g, p, r] * R[r, g, s]
    exp = np.zeros((n, n))
    for g in range(b2):
        for p in range(n // b2):
            for r in range(b1):
                for s in range(q1i):
                    exp[p * b2 + g, r * q1i + s] = w2[g, p, r] * w1[r, g, s]
    np.testing.assert_allclose(M, exp, rtol=1e-13, atol=1e-13)
    # the page's rearrangement (p k)(r s) -> k r p s: every (k, r) slice rank 1
    T = M.reshape(n // b2, b2, b1, q1i).transpose(1, 2, 0, 3)
    for k in range(b2):
        for r in range(b1):
            sv = np.linalg.svd(T[k, r], compute_uv=False)
            assert sv[1:].max(initial=0.0) <= 1e-12 * sv[0]


@pytest.mark.parametrize("n,b1,b2", [(16, 4, 4), (16, 2, 8), (16, 8, 2), (8, 2, 4), (8, 4, 2),
                                     (36, 6, 6), (24, 4, 6)])
def test_definition_c3_closed_form(n, b1, b2):
    check_closed_form(n, b1, b2)


@pytest.mark.parametrize("inp,out,b1,b2,rank", [(64, 32, 4, 4, 2), (48, 96, 2, 4, 12),
                                                (16, 64, 2, 2, 8), (24, 48, 3, 4, 4)])
def test_rectangular_slice_rank(inp, out, b1, b2, rank):
    # generalisation of the rank-1 slices: for block pair (g, r) the (p, s)
    # slice sums over the t with t*b2+g inside R-block r: mid/(b1*b2) terms
    w1, w2 = _rand_factors(inp, out, b1, b2, seed=5)
    M = O.monarch_matrix(w1, w2, inp, out)
    s = O.derive_sizes(inp, out, b1, b2)
    T = M.reshape(s["q2o"], b2, b1, s["q1i"]).transpose(1, 2, 0, 3)
    for g in range(b2):
        for r in range(b1):
            sv = np.linalg.svd(T[g, r], compute_uv=False)
            assert sv[rank - 1] > 1e-8 * sv[0]
            if rank < len(sv):
                assert sv[rank:].max() <= 1e-11 * sv[0]


# --------------------------------------------------------------------------
# P3: parameter counts
# --------------------------------------------------------------------------

def test_param_counts_definition_vs_code():
    # Definition C.3 (R: b blocks, L: n/b blocks) has n^2/b + n*b entries;
    # the MonarchLinear code (both factors b blocks) has 2 n^2 / b.
    for n, b in [(16, 2), (16, 4), (64, 4), (1024, 32), (16384, 128)]:
        assert O.param_count(n, n, b, n // b) == n * n // b + n * b
        assert O.param_count(n, n, b, b) == 2 * n * n // b
        assert O.param_count(n, n, b, b) < n * n or b <= 2


def test_param_counts_workloads():
    expected = {
        "tiny_square_n16_b4": 128,
        "square_n1024_b32": 65_536,
        "gpt2_ffn_up_768x3072_nb4": 2_949_120,
        "recsys_mlp_10000x1024x512_nb4_b1000": 3_018_752,
        "recsys_mlp_10000x1024x512_nb16_b1000": 754_688,
        "square_n16384_b128": 4_194_304,
    }
    for name, cnt in expected.items():
        w = S.WORKLOADS[name]
        assert sum(O.param_count(l.in_features, l.out_features, l.nblocks1, l.nblocks2)
                   for l in w.layers) == cnt
        assert w.params == cnt


def test_factor_shapes_follow_monarchlinear_rule():
    # MonarchLinear (Definition C.3 thread), branch in_ext >= out_ext:
    # blkdiag1 (nb, out_blk, in_blk), blkdiag2 (nb, out_blk, out_blk)
    for inp, out, nb in [(16, 16, 4), (1024, 1024, 32), (10000, 1024, 4), (1024, 512, 16)]:
        in_blk, out_blk = -(-inp // nb), -(-out // nb)
        w1, w2 = _rand_factors(inp, out, nb, nb)
        assert w1.shape == (nb, out_blk, in_blk)
        assert w2.shape == (nb, out_blk, out_blk)


# --------------------------------------------------------------------------
# P4: identity and permutation blocks
# --------------------------------------------------------------------------

@pytest.mark.parametrize("inp,out,b1,b2", [(16, 16, 4, 4), (16, 16, 2, 8), (64, 64, 8, 8)])
def test_identity_blocks_give_identity(inp, out, b1, b2):
    s = O.derive_sizes(inp, out, b1, b2)
    w1 = np.stack([np.eye(s["q1o"], s["q1i"])] * b1)
    w2 = np.stack([np.eye(s["q2o"], s["q2i"])] * b2)
    assert np.array_equal(O.monarch_matrix(w1, w2, inp, out), np.eye(out, inp))


@pytest.mark.parametrize("inp,out,b1,b2", [(16, 16, 4, 4), (64, 64, 8, 8), (32, 32, 4, 8)])
def test_shift_blocks_give_known_permutation(inp, out, b1, b2):
    s = O.derive_sizes(inp, out, b1, b2)
    a, c = 1, 3
    sh1 = np.roll(np.eye(s["q1i"]), a, axis=1)      # (sh1 x)[k] = x[(k + a) % q]
    sh2 = np.roll(np.eye(s["q2i"]), c, axis=1)
    M = O.monarch_matrix(np.stack([sh1] * b1), np.stack([sh2] * b2), inp, out)
    assert set(np.unique(M)) <= {0.0, 1.0}
    assert np.all(M.sum(0) == 1) and np.all(M.sum(1) == 1)
    # follow one unit through the index maps by hand
    for j_in in range(inp):
        r, si = divmod(j_in, s["q1i"])
        k = (si - a) % s["q1i"]                     # Z position inside block r
        z = r * s["q1o"] + k
        t, g = divmod(z, b2)                         # W[g*q2i + t] = Z[t*b2 + g]
        p = (t - c) % s["q2i"]
        assert M[p * b2 + g, j_in] == 1.0


# --------------------------------------------------------------------------
# P5: multiply applied to the identity returns the whole matrix
# --------------------------------------------------------------------------

def test_eye8_example():
    for lhs, rhs in _read_golden("eye8_example.txt"):
        n, nb, bs = (int(v) for v in lhs)
        rows, cols = (int(v) for v in rhs.split())
        w1, w2 = _rand_factors(n, n, nb, nb, seed=6)
        assert w1.shape == (nb, bs, bs) and w2.shape == (nb, bs, bs)
        Y = O.forward(np.eye(n), w1, w2, n, n)
        assert Y.shape == (rows, cols)
        np.testing.assert_allclose(Y, O.monarch_matrix(w1, w2, n, n).T, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# P6 / P10: brute force by loops on tiny inputs
# --------------------------------------------------------------------------

def _loop_forward(x, w1, w2, inp, out):
    """Pure-Python loops over single units, following the stage index maps."""
    s = O.derive_sizes(inp, out, w1.shape[0], w2.shape[0])
    b1, b2 = s["b1"], s["b2"]
    z = [0.0] * s["mid"]
    for r in range(b1):
        for k in range(s["q1o"]):
            acc = 0.0
            for si in range(s["q1i"]):
                acc += float(w1[r][k][si]) * float(x[r * s["q1i"] + si])
            z[r * s["q1o"] + k] = acc
    y = [0.0] * out
    for g in range(b2):
        for p in range(s["q2o"]):
            acc = 0.0
            for t in range(s["q2i"]):
                acc += float(w2[g][p][t]) * z[t * b2 + g]
            y[p * b2 + g] = acc
    return np.array(y)


@pytest.mark.parametrize("inp,out,b1,b2", [(16, 16, 4, 4), (8, 8, 2, 2), (8, 8, 2, 4),
                                           (12, 24, 3, 2), (16, 8, 4, 2), (6, 6, 1, 3)])
def test_loop_brute_force(inp, out, b1, b2):
    w1, w2 = _rand_factors(inp, out, b1, b2, seed=7)
    X = _rng(8).standard_normal((3, inp))
    Y = O.forward(X, w1, w2, inp, out)
    for b in range(3):
        np.testing.assert_allclose(Y[b], _loop_forward(X[b], w1, w2, inp, out), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P7: density
# --------------------------------------------------------------------------

@pytest.mark.parametrize("inp,out,b1,b2", [(16, 16, 4, 4), (64, 32, 4, 4), (48, 96, 2, 4),
                                           (30, 12, 3, 4)])
def test_dense_when_blocks_cover(inp, out, b1, b2):
    assert b1 * b2 <= out
    w1, w2 = _rand_factors(inp, out, b1, b2, seed=9)
    assert np.all(O.monarch_matrix(w1, w2, inp, out) != 0.0)


# --------------------------------------------------------------------------
# P8 / P9: backward pass
# --------------------------------------------------------------------------

CASES = [(16, 16, 4, 4, False), (16, 16, 2, 8, False), (24, 48, 3, 4, False), (64, 32, 4, 4, True),
         (20, 20, 5, 4, True)]


def check_euler(inp, out, b1, b2, relu, seed=10):
    w1, w2 = _rand_factors(inp, out, b1, b2, seed=seed)
    r = _rng(seed + 1)
    X = r.standard_normal((7, inp))
    dY = r.standard_normal((7, out))
    Y = O.forward(X, w1, w2, inp, out, relu=relu)
    dX, dw1, dw2 = O.backward(dY, X, w1, w2, inp, out, relu=relu, y=Y)
    e = np.vdot(dY, Y)
    # Y is positively homogeneous of degree 1 in each of X, R and L
    for v in (np.vdot(dX, X), np.vdot(dw1, w1), np.vdot(dw2, w2)):
        assert abs(v - e) <= 1e-11 * (abs(e) + np.abs(dY).sum())


@pytest.mark.parametrize("inp,out,b1,b2,relu", CASES)
def test_euler_identities(inp, out, b1, b2, relu):
    check_euler(inp, out, b1, b2, relu)


def check_finite_differences(inp, out, b1, b2, relu, seed=11):
    w1, w2 = _rand_factors(inp, out, b1, b2, seed=seed)
    r = _rng(seed + 1)
    X = r.standard_normal((4, inp))
    dY = r.standard_normal((4, out))

    def f(X_, w1_, w2_):
        return np.vdot(dY, O.forward(X_, w1_, w2_, inp, out, relu=relu))

    dX, dw1, dw2 = O.backward(dY, X, w1, w2, inp, out, relu=relu)
    h = 1e-6
    pick = _rng(seed + 2)
    for name, arr, grad in (("x", X, dX), ("w1", w1, dw1), ("w2", w2, dw2)):
        for _ in range(6):
            idx = tuple(pick.integers(0, d) for d in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = dict(x=X, w1=w1, w2=w2)
            args_m = dict(x=X, w1=w1, w2=w2)
            args_p[name], args_m[name] = ap, am
            fd = (f(args_p["x"], args_p["w1"], args_p["w2"]) - f(args_m["x"], args_m["w1"], args_m["w2"])) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("inp,out,b1,b2,relu", CASES)
def test_finite_differences(inp, out, b1, b2, relu):
    check_finite_differences(inp, out, b1, b2, relu)


def check_mlp_chain(seed=20):
    """Central finite differences through the two-layer chain with a ReLU
    between (the recommender MLP of the "efficiency testing numbers" thread,
    shapes scaled down): dX and sampled entries of both layers' dw1 and dw2.
    The weight gradients of each layer must see that layer's own input (the
    previous layer's post-ReLU output) and the gradient arriving from the
    layer above, masked where the ReLU was inactive."""
    l1 = _rand_factors(40, 16, 4, 4, seed=seed) + (40, 16, True)
    l2 = _rand_factors(16, 8, 4, 4, seed=seed + 1) + (16, 8, False)
    layers = [l1, l2]
    X = _rng(seed + 2).random((3, 40))
    dY = _rng(seed + 3).standard_normal((3, 8))
    dX, grads = O.mlp_backward(dY, X, layers)
    h = 1e-6

    def f(Xv, lay):
        return np.vdot(dY, O.mlp_forward(Xv, lay)[0])

    def fd_x(idx):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += h
        Xm[idx] -= h
        return (f(Xp, layers) - f(Xm, layers)) / (2 * h)

    def fd_w(li, wi, idx):
        def with_shift(d):
            lay = [list(l) for l in layers]
            w = lay[li][wi].copy()
            w[idx] += d
            lay[li][wi] = w
            return [tuple(l) for l in lay]
        return (f(X, with_shift(h)) - f(X, with_shift(-h))) / (2 * h)

    for idx in [(0, 0), (1, 17), (2, 39)]:
        fd = fd_x(idx)
        assert abs(fd - dX[idx]) < 1e-6 * (1 + abs(fd)), ("x", idx, fd, dX[idx])
    pick = _rng(seed + 4)
    for li in range(2):
        for wi in range(2):
            g = grads[li][wi]
            for _ in range(8):
                idx = tuple(int(pick.integers(0, d)) for d in g.shape)
                fd = fd_w(li, wi, idx)
                assert abs(fd - g[idx]) < 1e-6 * (1 + abs(fd)), (li, wi, idx, fd, g[idx])
    # every weight gradient is exercised (not all zero by a dead ReLU)
    assert all(np.abs(g).max() > 1e-3 for lg in grads for g in lg)


def test_mlp_chain_matches_finite_differences():
    check_mlp_chain(20)
    check_mlp_chain(50)


def test_sampled_helpers_match_full():
    inp, out, b1, b2 = 48, 96, 2, 4
    w1, w2 = _rand_factors(inp, out, b1, b2, seed=30)
    r = _rng(31)
    X = r.standard_normal((9, inp))
    dY = r.standard_normal((9, out))
    for relu in (False, True):
        Y = O.forward(X, w1, w2, inp, out, relu=relu)
        dX, dw1, dw2 = O.backward(dY, X, w1, w2, inp, out, relu=relu, y=Y)
        for sparse in (False, True):
            fac = O.dense_factors(w1, w2, inp, out, sparse=sparse)
            np.testing.assert_allclose(O.forward_rows(X[[2, 5]], w1, w2, inp, out, relu=relu, factors=fac),
                                       Y[[2, 5]], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(O.backward_dx_rows(dY[[1, 8]], w1, w2, inp, out, factors=fac,
                                                          y_rows=Y[[1, 8]], relu=relu),
                                       dX[[1, 8]], rtol=1e-12, atol=1e-12)
            rks = [(0, 3, 5), (1, 47, 23)]
            gpt = [(0, 0, 0), (3, 23, 11)]
            er, el = O.weight_grad_entries(dY, X, w1, w2, inp, out, rks, gpt, factors=fac, y=Y, relu=relu)
            np.testing.assert_allclose(er, [dw1[i] for i in rks], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(el, [dw2[i] for i in gpt], rtol=1e-11, atol=1e-12)


def test_row_errors():
    ref = np.array([[3.0, 4.0], [0.0, 10.0], [1.0, 0.0]])
    a = ref.copy()
    assert O.max_row_rel_error(a, ref) == 0.0 and O.parity_error(a, ref) == 0.0
    # one row off by 10% of its own norm: the worst row reports 0.1 while the
    # whole-tensor Frobenius error is diluted by the other rows
    a[2] = [1.1, 0.0]
    assert abs(O.max_row_rel_error(a, ref) - 0.1) < 1e-12
    assert O.rel_frobenius(a, ref) < 0.02
    assert abs(O.parity_error(a, ref) - 0.1) < 1e-12
    # a zeroed row fails the row bound whatever the other rows hold
    big = np.ones((4113, 8))
    z = big.copy()
    z[17] = 0.0
    assert O.rel_frobenius(z, big) < 0.02 and O.max_row_rel_error(z, big) == 1.0
    # a reference row of zeros is measured against the floor (1e-3 of the RMS row norm)
    r0 = np.array([[1.0, 0.0], [0.0, 0.0]])
    rms = np.linalg.norm(r0) / np.sqrt(2)
    e = O.max_row_rel_error(np.array([[1.0, 0.0], [1e-6, 0.0]]), r0)
    assert abs(e - 1e-6 / (1e-3 * rms)) < 1e-12
    # weight-gradient blocks: rows along the last axis
    g = np.arange(24, dtype=float).reshape(2, 3, 4) + 1
    h = g.copy()
    h[1, 2, 3] *= 1.5
    row = g[1, 2]
    assert abs(O.max_row_rel_error(h, g) - 0.5 * row[3] / np.linalg.norm(row)) < 1e-12


def test_row_errors_against_absolute_scale():
    # a row whose terms cancel: ref = 1 - 0.999, scale = 1 + 0.999
    ref = np.array([[0.001, 5.0]])
    scale = np.array([[1.999, 5.0]])
    a = ref + np.array([[1e-3, 0.0]])
    assert abs(O.max_row_rel_error(a, ref, scale) - 1e-3 / np.linalg.norm(scale)) < 1e-15
    assert O.max_row_rel_error(a, ref) > O.max_row_rel_error(a, ref, scale)
    # the scale of a sum is the same sum over magnitudes: for the Monarch
    # product it is the oracle run on |X|, |w1|, |w2|
    w1, w2 = _rand_factors(16, 16, 4, 4, seed=3)
    x = _rng(4).standard_normal((5, 16))
    sc = O.forward(np.abs(x), np.abs(w1), np.abs(w2), 16, 16)
    assert np.all(sc >= np.abs(O.forward(x, w1, w2, 16, 16)) - 1e-12)
    assert O.parity_error(O.forward(x, w1, w2, 16, 16), O.forward(x, w1, w2, 16, 16), sc) == 0.0


def test_rel_frobenius():
    a = np.array([3.0, 4.0])
    assert O.rel_frobenius(a, a) == 0.0
    assert abs(O.rel_frobenius(a * 1.1, a) - 0.1) < 1e-12
    assert O.rel_frobenius(np.zeros(2), np.zeros(2)) == 0.0


# --------------------------------------------------------------------------
# P11: bfloat16 rounding used for the inputs
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    r = _rng(40)
    a = np.concatenate([
        r.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38], dtype=np.float32),
        # exact ties: mantissa low half = 0x8000 with even and odd kept bit
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x7F7FFFFF], dtype=np.uint32).view(np.float32),
    ])
    mine = S.round_to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(mine.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(S.round_to_bf16(np.array([np.nan], dtype=np.float32)))[0]
    bits = S.bf16_bits(mine)
    assert np.array_equal(S.bf16_bits_to_f32(bits).view(np.uint32), mine.view(np.uint32))


def test_inputs_are_seeded_and_scaled():
    w = S.WORKLOADS["tiny_square_n16_b4"]
    a = S.make_layer_inputs(w)
    b = S.make_layer_inputs(w)
    for k in a:
        assert np.array_equal(a[k], b[k])
    big = S.draw(S.seed_for(1, 0), (4096, 64), "normal", 0.25)
    assert abs(big.var() - 0.25) < 0.01
    u = S.draw(1, (10000,), "uniform")
    assert u.min() >= 0.0 and u.max() < 1.0
    wb = S.make_layer_inputs(S.WORKLOADS["square_n1024_b32"], batch=4)
    assert np.array_equal(S.round_to_bf16(wb["w1"]), wb["w1"])


# --------------------------------------------------------------------------
# planted mistakes: each slip must fail a pin
# --------------------------------------------------------------------------

def _expect_fail(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_planted_transposed_permutation_is_caught(monkeypatch):
    orig = O.monarch_oracle.stride_permutation
    monkeypatch.setattr(O.monarch_oracle, "stride_permutation",
                        lambda mid, nb2, sparse=False: orig(mid, nb2, sparse).T)
    _expect_fail(check_closed_form, 16, 2, 8)


def test_planted_missing_output_permutation_is_caught(monkeypatch):
    monkeypatch.setattr(O.monarch_oracle, "output_permutation",
                        lambda out, nb2, sparse=False: np.eye(out))
    _expect_fail(check_closed_form, 16, 4, 4)


def test_planted_transposed_block_is_caught(monkeypatch):
    orig = O.monarch_oracle.block_diag_dense
    monkeypatch.setattr(O.monarch_oracle, "block_diag_dense",
                        lambda blocks, sparse=False: orig(np.swapaxes(blocks, 1, 2), sparse))
    _expect_fail(check_closed_form, 16, 4, 4)


def test_planted_permutation_in_wrong_place_is_caught(monkeypatch):
    # P applied after stage 2 instead of between the stages
    def bad_matrix(w1, w2, inp, out):
        Rd, Pm, Ld, Qo = O.dense_factors(w1, w2, inp, out)
        return Qo @ Pm @ Ld @ Rd
    monkeypatch.setattr(O.monarch_oracle, "monarch_matrix", bad_matrix)
    monkeypatch.setattr(O, "monarch_matrix", bad_matrix)
    _expect_fail(check_closed_form, 16, 4, 4)


def test_planted_backward_slip_is_caught(monkeypatch):
    orig = O.monarch_oracle.backward

    def bad_backward(*a, **k):
        dX, dw1, dw2 = orig(*a, **k)
        return dX, np.swapaxes(dw1, 1, 2) if dw1.shape[1] == dw1.shape[2] else dw1 * 0.5, dw2
    monkeypatch.setattr(O.monarch_oracle, "backward", bad_backward)
    monkeypatch.setattr(O, "backward", bad_backward)
    _expect_fail(check_finite_differences, 16, 16, 4, 4, False)
    _expect_fail(check_euler, 16, 16, 4, 4, False)


def test_planted_relu_mask_slip_is_caught(monkeypatch):
    orig = O.monarch_oracle.backward

    def no_mask(dy, x, w1, w2, inp, out, relu=False, y=None, factors=None):
        return orig(dy, x, w1, w2, inp, out, relu=False, y=None, factors=factors)
    monkeypatch.setattr(O, "backward", no_mask)
    _expect_fail(check_finite_differences, 64, 32, 4, 4, True)


def test_planted_mlp_wrong_activation_is_caught(monkeypatch):
    # layer 2's weight gradients computed from layer 1's pre-ReLU output
    # (the wrong activation) instead of its post-ReLU input
    def bad_mlp_backward(dy, x, layers):
        h = np.asarray(x, dtype=np.float64)
        acts, pre = [h], [h]
        for (w1, w2, fi, fo, relu) in layers:
            z = O.forward(h, w1, w2, fi, fo, relu=False)
            h = np.maximum(z, 0) if relu else z
            pre.append(z)
            acts.append(h)
        g = np.asarray(dy, dtype=np.float64)
        grads = [None] * len(layers)
        for i in range(len(layers) - 1, -1, -1):
            w1, w2, fi, fo, relu = layers[i]
            src = pre[i] if i > 0 else acts[i]
            _, dw1, dw2 = O.backward(g, src, w1, w2, fi, fo, relu=relu,
                                     y=acts[i + 1] if relu else None)
            g, _, _ = O.backward(g, acts[i], w1, w2, fi, fo, relu=relu,
                                 y=acts[i + 1] if relu else None)
            grads[i] = (dw1, dw2)
        return g, grads
    monkeypatch.setattr(O, "mlp_backward", bad_mlp_backward)
    _expect_fail(check_mlp_chain, 20)


def test_planted_mlp_unmasked_gradient_is_caught(monkeypatch):
    # layer 1's weight gradients taken from the gradient above the ReLU,
    # without its mask
    orig = O.monarch_oracle.backward

    def bad_backward(dy, x, w1, w2, inp, out, relu=False, y=None, factors=None):
        return orig(dy, x, w1, w2, inp, out, relu=False, factors=factors)
    monkeypatch.setattr(O.monarch_oracle, "backward", bad_backward)
    _expect_fail(check_mlp_chain, 20)
