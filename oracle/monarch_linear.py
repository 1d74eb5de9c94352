"""MonarchLinear shape variants: a plain fp64 CPU statement of the general
layer the library's *_ex entry points compute. TEST INFRASTRUCTURE ONLY (the
same rules as monarch_oracle: only tests/, the smoke check and the
benchmark's CPU leg use it; it shares no code with the HIP path).

What is computed
----------------
The MonarchLinear constructor quoted in the "Definition C.3" thread of the
scatterbrain issues page sizes its two block tensors from one block count nb:

    in_blksz  = ceil(in / nb),   in_ext  = nb * in_blksz
    out_blksz = ceil(out / nb),  out_ext = nb * out_blksz
    in_ext <  out_ext:  blkdiag1 (nb, in_blksz,  in_blksz),  blkdiag2 (nb, out_blksz, in_blksz)
    otherwise:          blkdiag1 (nb, out_blksz, in_blksz),  blkdiag2 (nb, out_blksz, out_blksz)

so the intermediate width is mid = in_ext for an expanding layer and
out_ext otherwise. The page prints no forward for the padded sizes; the
reading adopted (the plainest one the sizes support) is: the input is
zero-padded from in to in_ext features, the two-stage product runs at the
extended sizes, and the output keeps its first out features. With a bias
vector b (length out, added before the activation, as a drop-in for a linear
layer) the layer is

    Y = act( X · Mᵀ + b ),   M = T_out · Q_out · L · P · R · E_in      (out x in)

with E_in (in_ext x in) the zero-padding embedding, R (mid x in_ext) and L
(out_ext x mid) block-diagonal, P (mid x mid) the stride-nb2 permutation
(P z)[g*q2i + t] = z[t*nb2 + g], Q_out (out_ext x out_ext) its output
counterpart (Q v)[p*nb2 + g] = v[g*q2o + p] (not Pᵀ once mid != out), and
T_out (out x out_ext) the truncation. The general form takes nb1 and nb2
separately: q1i = ceil(in/nb1), q2o = ceil(out/nb2), q1o = mid/nb1,
q2i = mid/nb2.

Parity pins (tests/test_linear_oracle.py): the page's parameter shapes, the
reduction to the pinned square/rectangular oracle, a literal block-by-block
loop over the index maps, zero-padding and truncation invariants, bias
linearity, central finite differences and the multilinearity identities.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from .monarch_oracle import block_diag_dense


def linear_sizes(in_features: int, out_features: int, nblocks: int) -> Dict[str, int]:
    """Block sizes of the MonarchLinear constructor (one block count)."""
    if in_features <= 0 or out_features <= 0 or nblocks <= 0:
        raise ValueError("sizes must be positive")
    in_blksz = int(math.ceil(in_features / nblocks))
    out_blksz = int(math.ceil(out_features / nblocks))
    in_ext, out_ext = in_blksz * nblocks, out_blksz * nblocks
    mid = in_ext if in_ext < out_ext else out_ext
    return general_sizes(in_features, out_features, mid, nblocks, nblocks)


def general_sizes(in_features: int, out_features: int, mid: int, nblocks1: int,
                  nblocks2: int) -> Dict[str, int]:
    """Sizes with an explicit intermediate width (mid divisible by both block
    counts); in and out are padded up to whole blocks."""
    if min(in_features, out_features, mid, nblocks1, nblocks2) <= 0:
        raise ValueError("sizes must be positive")
    if mid % nblocks1 or mid % nblocks2:
        raise ValueError("mid must be divisible by both block counts")
    q1i = -(-in_features // nblocks1)
    q2o = -(-out_features // nblocks2)
    return dict(inp=in_features, out=out_features, mid=mid, b1=nblocks1, b2=nblocks2,
                q1i=q1i, q1o=mid // nblocks1, q2i=mid // nblocks2, q2o=q2o,
                in_ext=q1i * nblocks1, out_ext=q2o * nblocks2)


def _perm(rows, cols, n):
    A = np.zeros((n, n))
    A[rows, cols] = 1.0
    return A


def dense_factors_ex(w1: np.ndarray, w2: np.ndarray, in_features: int, out_features: int,
                     mid: int):
    """(E_in, Rd, Pm, Ld, Qo, T_out) with M = T_out·Qo·Ld·Pm·Rd·E_in."""
    nb1, nb2 = w1.shape[0], w2.shape[0]
    s = general_sizes(in_features, out_features, mid, nb1, nb2)
    if w1.shape != (nb1, s["q1o"], s["q1i"]) or w2.shape != (nb2, s["q2o"], s["q2i"]):
        raise ValueError("factor shapes do not match the sizes")
    E = np.zeros((s["in_ext"], in_features))
    E[np.arange(in_features), np.arange(in_features)] = 1.0       # zero-pad at the end
    Rd = block_diag_dense(w1)
    g, t = np.meshgrid(np.arange(nb2), np.arange(s["q2i"]), indexing="ij")
    Pm = _perm((g * s["q2i"] + t).ravel(), (t * nb2 + g).ravel(), mid)
    Ld = block_diag_dense(w2)
    g, p = np.meshgrid(np.arange(nb2), np.arange(s["q2o"]), indexing="ij")
    Qo = _perm((p * nb2 + g).ravel(), (g * s["q2o"] + p).ravel(), s["out_ext"])
    T = np.zeros((out_features, s["out_ext"]))
    T[np.arange(out_features), np.arange(out_features)] = 1.0     # keep the first out
    return E, Rd, Pm, Ld, Qo, T


def monarch_matrix_ex(w1, w2, in_features, out_features, mid) -> np.ndarray:
    """The dense out x in matrix of the padded/truncated layer, fp64."""
    E, Rd, Pm, Ld, Qo, T = dense_factors_ex(w1, w2, in_features, out_features, mid)
    return T @ Qo @ Ld @ Pm @ Rd @ E


def forward_ex(x, w1, w2, in_features, out_features, mid, bias=None, relu=False):
    """Y = act(X·Mᵀ + bias) through the dense factor chain (fp64)."""
    X = np.asarray(x, dtype=np.float64)
    E, Rd, Pm, Ld, Qo, T = dense_factors_ex(w1, w2, in_features, out_features, mid)
    Y = X @ E.T @ Rd.T @ Pm.T @ Ld.T @ Qo.T @ T.T
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float64)[None, :]
    if relu:
        Y = np.maximum(Y, 0.0)
    return Y


def backward_ex(dy, x, w1, w2, in_features, out_features, mid, bias=None, relu=False,
                y: Optional[np.ndarray] = None):
    """Gradients of sum(dY * Y) with respect to X, w1, w2 and the bias.

    With dY_eff = dY ⊙ 1[Y > 0] after a ReLU (derivative 0 at 0):
        dV = dY_eff·T_out·Qo,  dW = dV·Ld,  dZ = dW·Pm,  dX = dZ·Rd·E_in,
        dL[g] = block g of dVᵀ·W,  dR[r] = block r of dZᵀ·(X·E_inᵀ),
        dbias = column sums of dY_eff,
    with W = X·E_inᵀ·Rdᵀ·Pmᵀ stage 2's input. Returns (dX, dw1, dw2, dbias)."""
    X = np.asarray(x, dtype=np.float64)
    dY = np.asarray(dy, dtype=np.float64)
    nb1, nb2 = w1.shape[0], w2.shape[0]
    s = general_sizes(in_features, out_features, mid, nb1, nb2)
    E, Rd, Pm, Ld, Qo, T = dense_factors_ex(w1, w2, in_features, out_features, mid)
    if relu:
        if y is None:
            y = forward_ex(X, w1, w2, in_features, out_features, mid, bias, relu=True)
        dY = dY * (np.asarray(y, dtype=np.float64) > 0)
    Xe = X @ E.T
    W = Xe @ Rd.T @ Pm.T
    dV = dY @ T @ Qo
    dZ = dV @ Ld @ Pm
    dX = dZ @ Rd @ E
    q1o, q1i, q2o, q2i = s["q1o"], s["q1i"], s["q2o"], s["q2i"]
    dw2 = np.empty((nb2, q2o, q2i))
    for g in range(nb2):
        dw2[g] = dV[:, g * q2o:(g + 1) * q2o].T @ W[:, g * q2i:(g + 1) * q2i]
    dw1 = np.empty((nb1, q1o, q1i))
    for r in range(nb1):
        dw1[r] = dZ[:, r * q1o:(r + 1) * q1o].T @ Xe[:, r * q1i:(r + 1) * q1i]
    dbias = dY.sum(axis=0)
    return dX, dw1, dw2, dbias
