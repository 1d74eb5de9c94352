"""Dense -> Monarch projection oracle: a plain fp64 CPU statement of the
projection the GPU library computes. TEST INFRASTRUCTURE ONLY (the same rules
as monarch_oracle: only tests/, the smoke check and the benchmark's CPU leg
use it; it shares no code with the HIP path).

What is computed
----------------
The scatterbrain issues page ("projection" thread) describes the projection of
a dense matrix onto the Monarch factors in the Definition C.3 case: rearrange
M as '(p k) (r s) -> k r p s' and fit each (k, r) slice, a p x s matrix, on
its own; the Monarch paper's abstract calls the result an analytical optimal
solution. In this library's notation (w1 = R [b1, q1o, q1i], w2 = L
[b2, q2o, q2i], mid = out), the case is out = b1 * b2, so q1o = b2 and q2i = b1,
and the Monarch matrix has entries

    M[p*b2 + g, r*q1i + s] = L[g, p, r] * R[r, g, s],

i.e. the (k = g, r) slice over (p, s) is the outer product of L[g, :, r] and
R[r, g, :]. Every (L, R) pair touches its own slice only, so the
Frobenius-nearest Monarch matrix takes, slice by slice, the nearest rank-one
matrix: sigma * u * v^T from the slice's top singular triple (Eckart-Young).
The factors are split evenly, L[g, :, r] = sqrt(sigma) u and
R[r, g, :] = sqrt(sigma) v, with the sign fixed so that the entry of largest
magnitude of R[r, g, :] (the first one on ties) is positive.

Parity pins (tests/test_projection_oracle.py): exact reproduction of Monarch
inputs, optimality against perturbed and random factors, idempotence, the
rank-one slice structure of the page's rearrangement, and orthogonality of
the residual to the fit.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def projection_applies(in_features: int, out_features: int, nblocks1: int, nblocks2: int) -> bool:
    """The Definition C.3 case: out = nblocks1 * nblocks2 and in % nblocks1 == 0."""
    return (nblocks1 > 0 and nblocks2 > 0 and in_features % nblocks1 == 0
            and out_features == nblocks1 * nblocks2)


def slices(m: np.ndarray, in_features: int, out_features: int, nblocks1: int,
           nblocks2: int) -> np.ndarray:
    """The page's rearrangement '(p k) (r s) -> k r p s' with k = nblocks2 and
    r = nblocks1: slices[g, r, p, s] = M[p*b2 + g, r*q1i + s]."""
    b1, b2 = nblocks1, nblocks2
    q1i, q2o = in_features // b1, out_features // b2
    m = np.asarray(m, dtype=np.float64).reshape(q2o, b2, b1, q1i)
    return m.transpose(1, 2, 0, 3)


def fit_slice(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Nearest rank-one matrix of one p x s slice as (l, r) with l r^T the fit:
    l = sqrt(sigma) u, r = sqrt(sigma) v from the top singular triple, signed so
    that the entry of largest magnitude of r (the first on ties) is positive."""
    u, sv, vt = np.linalg.svd(np.asarray(a, dtype=np.float64), full_matrices=False)
    sigma = sv[0]
    uu, vv = u[:, 0], vt[0, :]
    j = int(np.argmax(np.abs(vv)))
    if vv[j] < 0:
        uu, vv = -uu, -vv
    return np.sqrt(sigma) * uu, np.sqrt(sigma) * vv


def project(m: np.ndarray, in_features: int, out_features: int, nblocks1: int,
            nblocks2: int) -> Tuple[np.ndarray, np.ndarray]:
    """Nearest Monarch factors (w1 = R, w2 = L) of a dense out x in matrix."""
    if not projection_applies(in_features, out_features, nblocks1, nblocks2):
        raise ValueError("projection needs out_features = nblocks1 * nblocks2 and "
                         "in_features divisible by nblocks1")
    b1, b2 = nblocks1, nblocks2
    q1i, q2o = in_features // b1, out_features // b2
    sl = slices(m, in_features, out_features, b1, b2)
    w1 = np.zeros((b1, b2, q1i))        # R[r, g, s]  (q1o = b2)
    w2 = np.zeros((b2, q2o, b1))        # L[g, p, r]  (q2i = b1)
    for g in range(b2):
        for r in range(b1):
            w2[g, :, r], w1[r, g, :] = fit_slice(sl[g, r])
    return w1, w2
