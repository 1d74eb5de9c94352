"""DYAD-style layer: a plain fp64 CPU statement of what the library's
monarch_dyad_* entry points compute. TEST INFRASTRUCTURE ONLY (same rules as
monarch_oracle; it shares no code with the HIP path).

What is computed
----------------
The DYAD page (abstract) describes a replacement for a dense linear layer
whose weight matrix is the sum of two matrices, each a permutation of a
block-sparse matrix and each stored as a 3D tensor, so that the product with
the input costs rows x cols / (number of blocks). Reading adopted (the
plainest one the abstract supports, with the permutation this library
already uses for Monarch): with nb blocks, qi = in / nb and qo = out / nb,

    M = BD(A) + Q_out · BD(B) · P_in            (out x in),   Y = X · Mᵀ,

  * BD(A): block-diagonal, block r = A[r] (qo x qi) on contiguous features;
  * P_in: the stride permutation (P x)[g*qi + t] = x[t*nb + g] (the
    reshape-transpose of the "hypercube" thread of the scatterbrain issues
    page), Q_out: its output counterpart (Q v)[p*nb + g] = v[g*qo + p];
  * so B[g] connects the inputs t*nb + g to the outputs p*nb + g.

A and B are stored as [nb, qo, qi]. The backward pass is the chain rule:
dX = dY·M, dA[r] = block r of dYᵀ·X, dB[g] = block g of (dY·Q_out)ᵀ·(X·P_inᵀ).

Parity pins (tests/test_dyad_oracle.py): a literal loop over the index maps,
the A = 0 case against the pinned Monarch oracle (identity R blocks), the
exact nonzero pattern (contiguous blocks or equal residues mod nb), the
parameter count, finite differences and the multilinearity identities.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .monarch_oracle import block_diag_dense, output_permutation, stride_permutation


def dyad_sizes(in_features: int, out_features: int, nblocks: int) -> Dict[str, int]:
    if nblocks <= 0 or in_features <= 0 or out_features <= 0:
        raise ValueError("sizes must be positive")
    if in_features % nblocks or out_features % nblocks:
        raise ValueError("in and out must be divisible by the block count")
    return dict(inp=in_features, out=out_features, nb=nblocks, qi=in_features // nblocks,
                qo=out_features // nblocks)


def param_count(in_features: int, out_features: int, nblocks: int) -> int:
    s = dyad_sizes(in_features, out_features, nblocks)
    return 2 * s["nb"] * s["qo"] * s["qi"]


def dyad_matrix(wa: np.ndarray, wb: np.ndarray, in_features: int, out_features: int) -> np.ndarray:
    s = dyad_sizes(in_features, out_features, np.asarray(wa).shape[0])
    shape = (s["nb"], s["qo"], s["qi"])
    if np.asarray(wa).shape != shape or np.asarray(wb).shape != shape:
        raise ValueError("factor shapes do not match the sizes")
    Pi = stride_permutation(in_features, s["nb"])
    Qo = output_permutation(out_features, s["nb"])
    return block_diag_dense(wa) + Qo @ block_diag_dense(wb) @ Pi


def forward(x, wa, wb, in_features, out_features):
    return np.asarray(x, dtype=np.float64) @ dyad_matrix(wa, wb, in_features, out_features).T


def backward(dy, x, wa, wb, in_features, out_features):
    """Returns (dX, dA, dB)."""
    X = np.asarray(x, dtype=np.float64)
    dY = np.asarray(dy, dtype=np.float64)
    s = dyad_sizes(in_features, out_features, np.asarray(wa).shape[0])
    nb, qi, qo = s["nb"], s["qi"], s["qo"]
    dX = dY @ dyad_matrix(wa, wb, in_features, out_features)
    Pi = stride_permutation(in_features, nb)
    Qo = output_permutation(out_features, nb)
    dYq = dY @ Qo            # gradient of BD(B)'s output (block-major)
    Xp = X @ Pi.T            # BD(B)'s input (block-major)
    dA = np.empty((nb, qo, qi))
    dB = np.empty((nb, qo, qi))
    for r in range(nb):
        dA[r] = dY[:, r * qo:(r + 1) * qo].T @ X[:, r * qi:(r + 1) * qi]
        dB[r] = dYq[:, r * qo:(r + 1) * qo].T @ Xp[:, r * qi:(r + 1) * qi]
    return dX, dA, dB
