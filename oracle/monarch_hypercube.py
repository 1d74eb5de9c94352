"""k-factor ("hypercube") Monarch: a plain fp64 CPU statement of the layer the
library's monarch_hyper_* entry points compute. TEST INFRASTRUCTURE ONLY (same
rules as monarch_oracle; it shares no code with the HIP path).

What is computed
----------------
The "hypercube" thread of the scatterbrain issues page views the N units of
a layer as a lattice of shape [n_1, ..., n_k] (its example: 12288 = 16 * 24 *
32) and applies one round per dimension: round j multiplies along axis j,
with its own n_j x n_j matrix for every combination of the other axes' indices
(N / n_j matrices: 768, 512 and 384 in the example). The two-factor Monarch is
the case k = 2 (its 4-unit example: the two products run over the columns and
the rows of a 2 x 2 square).

Readings adopted where the page is silent:
  * the lattice is row-major: unit u has multi-index (a_1, ..., a_k) with
    u = ((a_1 * n_2 + a_2) * n_3 + ...) * n_k + a_k;
  * round j's matrices are indexed by the other axes' indices flattened
    row-major in axis order (f), stored as w_j [N / n_j, n_j, n_j] with
    w_j[f][o, i] the weight from position i to position o along axis j
    (the (out, in) block layout of the two-factor factors);
  * the rounds run in axis order j = 1, ..., k, as the page lists them.

With F_j the N x N matrix of round j, the layer is y = F_k ... F_1 x per row,
Y = X · Mᵀ with M = F_k ... F_1. The backward pass is the chain rule through
the rounds: with x_j = F_j x_{j-1} (x_0 = x) and g_k = dY,
    g_{j-1} = g_j · F_j,   dw_j[f] = sum over rows of g_j[fiber f]ᵀ x_{j-1}[fiber f].

Parity pins (tests/test_hypercube_oracle.py): the page's matrix counts, the
reduction of k = 2 to the pinned two-factor oracle under the lattice
transpose, a literal loop over multi-indices, identity and permutation
blocks, central finite differences and the multilinearity identities.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def check_dims(dims: Sequence[int]) -> Tuple[int, ...]:
    dims = tuple(int(d) for d in dims)
    if not dims or any(d <= 0 for d in dims):
        raise ValueError("lattice dimensions must be positive")
    return dims


def fiber_positions(dims: Sequence[int], j: int) -> np.ndarray:
    """pos[f, a]: flat unit index of position a along axis j in fiber f (the
    other axes' indices flattened row-major)."""
    dims = check_dims(dims)
    idx = np.arange(int(np.prod(dims))).reshape(dims)
    moved = np.moveaxis(idx, j, -1)          # other axes in order, axis j last
    return moved.reshape(-1, dims[j])


def weight_shapes(dims: Sequence[int]) -> List[Tuple[int, int, int]]:
    dims = check_dims(dims)
    n = int(np.prod(dims))
    return [(n // d, d, d) for d in dims]


def param_count(dims: Sequence[int]) -> int:
    return sum(a * b * c for a, b, c in weight_shapes(dims))


def round_matrix(w: np.ndarray, dims: Sequence[int], j: int) -> np.ndarray:
    """Dense N x N matrix F_j of round j."""
    dims = check_dims(dims)
    n = int(np.prod(dims))
    pos = fiber_positions(dims, j)
    w = np.asarray(w, dtype=np.float64)
    if w.shape != (pos.shape[0], dims[j], dims[j]):
        raise ValueError("weight shape does not match the lattice")
    F = np.zeros((n, n))
    for f in range(pos.shape[0]):
        F[np.ix_(pos[f], pos[f])] = w[f]
    return F


def hyper_matrix(ws: Sequence[np.ndarray], dims: Sequence[int]) -> np.ndarray:
    """M = F_k ... F_1 (N x N)."""
    dims = check_dims(dims)
    M = np.eye(int(np.prod(dims)))
    for j, w in enumerate(ws):
        M = round_matrix(w, dims, j) @ M
    return M


def forward(x, ws, dims, keep: bool = False):
    """Y = X · Mᵀ through the rounds (fp64); keep=True also returns
    [x_0, x_1, ..., x_k]."""
    dims = check_dims(dims)
    if len(ws) != len(dims):
        raise ValueError("one weight tensor per lattice dimension")
    h = np.asarray(x, dtype=np.float64)
    acts = [h]
    for j, w in enumerate(ws):
        h = h @ round_matrix(w, dims, j).T
        acts.append(h)
    return (h, acts) if keep else h


def backward(dy, x, ws, dims):
    """Gradients of sum(dY * Y) with respect to X and every round's weights.
    Returns (dX, [dw_1, ..., dw_k])."""
    dims = check_dims(dims)
    _, acts = forward(x, ws, dims, keep=True)
    g = np.asarray(dy, dtype=np.float64)
    grads = [None] * len(dims)
    for j in range(len(dims) - 1, -1, -1):
        pos = fiber_positions(dims, j)
        xin = acts[j]
        dw = np.empty((pos.shape[0], dims[j], dims[j]))
        for f in range(pos.shape[0]):
            dw[f] = g[:, pos[f]].T @ xin[:, pos[f]]
        grads[j] = dw
        g = g @ round_matrix(ws[j], dims, j)
    return g, grads


def forward_fibers(x, ws, dims, keep: bool = False):
    """The same rounds without dense N x N matrices: gather every fiber of
    axis j, multiply by its matrix, scatter back (for large lattices)."""
    dims = check_dims(dims)
    h = np.asarray(x, dtype=np.float64)
    acts = [h]
    for j, w in enumerate(ws):
        pos = fiber_positions(dims, j)
        out = np.empty_like(h)
        out[:, pos] = np.einsum("bfi,foi->bfo", h[:, pos], np.asarray(w, dtype=np.float64))
        h = out
        acts.append(h)
    return (h, acts) if keep else h


def backward_fibers(dy, x, ws, dims):
    """backward() evaluated fiber by fiber (no dense matrices)."""
    dims = check_dims(dims)
    _, acts = forward_fibers(x, ws, dims, keep=True)
    g = np.asarray(dy, dtype=np.float64)
    grads = [None] * len(dims)
    for j in range(len(dims) - 1, -1, -1):
        pos = fiber_positions(dims, j)
        w = np.asarray(ws[j], dtype=np.float64)
        gf, xf = g[:, pos], acts[j][:, pos]
        grads[j] = np.einsum("bfo,bfi->foi", gf, xf)
        gin = np.empty_like(g)
        gin[:, pos] = np.einsum("bfo,foi->bfi", gf, w)
        g = gin
    return g, grads
