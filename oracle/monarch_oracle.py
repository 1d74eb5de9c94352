"""Monarch multiply oracle: a plain, slow, fp64 CPU statement of what the
library computes. TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or call this module. The GPU library never routes through it, and this
module shares no code with the HIP path (it imports nothing from the package).

What is computed
----------------
A Monarch matrix is a product of two block-diagonal matrices up to a
permutation of rows and columns (Monarch paper, abstract; scatterbrain issues
page, "Definition C.3" thread). The library's operator, as a linear layer on
row-major activations, is

    M = Q_out · L · P · R          (out x in),      y = M x   per row,
    Y = X · Mᵀ                      (batch x out),

with the factors materialised here as explicit dense matrices:

  * R (mid x in), block-diagonal with nblocks1 blocks of shape (mid/nb1, in/nb1);
    block r is w1[r] (storage (nblocks, out_blk, in_blk), as the MonarchLinear
    parameters in the "Definition C.3" thread).
  * P (mid x mid), the stride permutation: reshape the length-mid vector to
    (mid/nb2, nb2) and transpose, i.e. (P z)[g*q2i + t] = z[t*nb2 + g]. For 4
    units and 2 blocks this gives [x0, x2, x1, x3] (scatterbrain issues page,
    "hypercube" thread, the 4-unit example).
  * L (out x mid), block-diagonal with nblocks2 blocks of shape (out/nb2, mid/nb2).
  * Q_out (out x out), the inverse stride permutation on the output:
    (Q_out v)[p*nb2 + g] = v[g*q2o + p]; with mid = out it is Pᵀ.

The intermediate width mid equals out_features (reading adopted for
rectangular layers; the GPT-2 FFN shape 768->3072 with stage-1 blocks 768x192
and stage-2 blocks 768x768 fixes it).

Everything is fp64; callers pass inputs already rounded to the workload's
storage precision. The backward pass is the chain rule through the dense
factor chain; the weight gradients are the diagonal blocks of the dense
gradients of the block-diagonal factors.

Parity pins (tests/test_oracle.py) tie every function here to facts fixed by
the pages or by mathematics; none is "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

try:  # sparse storage of the same factor matrices, used for full-size sampled checks
    import scipy.sparse as _sp
except Exception:  # pragma: no cover
    _sp = None


# ----------------------------------------------------------------------------
# sizes
# ----------------------------------------------------------------------------

def derive_sizes(in_features: int, out_features: int, nblocks1: int, nblocks2: int) -> Dict[str, int]:
    """Block sizes of the two factors (mid = out_features).

    R has nblocks1 blocks of (q1o x q1i), L has nblocks2 blocks of (q2o x q2i)
    (MonarchLinear parameter shapes, scatterbrain issues page, "Definition C.3"
    thread; non-divisible sizes are rejected rather than padded)."""
    mid = out_features
    for num, den in ((in_features, nblocks1), (mid, nblocks1), (mid, nblocks2), (out_features, nblocks2)):
        if den <= 0 or num <= 0 or num % den:
            raise ValueError(f"size {num} not divisible by block count {den}")
    return dict(inp=in_features, mid=mid, out=out_features, b1=nblocks1, b2=nblocks2,
                q1i=in_features // nblocks1, q1o=mid // nblocks1,
                q2i=mid // nblocks2, q2o=out_features // nblocks2)


def param_count(in_features: int, out_features: int, nblocks1: int, nblocks2: int) -> int:
    """Number of free parameters: the entries of the two block tensors."""
    s = derive_sizes(in_features, out_features, nblocks1, nblocks2)
    return s["b1"] * s["q1o"] * s["q1i"] + s["b2"] * s["q2o"] * s["q2i"]


# ----------------------------------------------------------------------------
# dense factor matrices
# ----------------------------------------------------------------------------

def block_diag_dense(blocks: np.ndarray, sparse: bool = False):
    """Dense (or scipy-sparse, same entries) block-diagonal matrix whose block
    b occupies rows [b*qo, (b+1)*qo) and columns [b*qi, (b+1)*qi)."""
    blocks = np.asarray(blocks, dtype=np.float64)
    nb, qo, qi = blocks.shape
    if sparse:
        return _sp.block_diag([blocks[b] for b in range(nb)], format="csr", dtype=np.float64)
    D = np.zeros((nb * qo, nb * qi), dtype=np.float64)
    for b in range(nb):
        D[b * qo:(b + 1) * qo, b * qi:(b + 1) * qi] = blocks[b]
    return D


def _perm_matrix(rows: np.ndarray, cols: np.ndarray, n: int, sparse: bool):
    if sparse:
        return _sp.csr_matrix((np.ones(n), (rows, cols)), shape=(n, n), dtype=np.float64)
    A = np.zeros((n, n), dtype=np.float64)
    A[rows, cols] = 1.0
    return A


def stride_permutation(mid: int, nblocks2: int, sparse: bool = False):
    """P with (P z)[g*q2i + t] = z[t*nblocks2 + g]: view z as a (q2i, nblocks2)
    row-major array and transpose it (the 4-unit example of the "hypercube"
    thread gives [x0, x2, x1, x3])."""
    q2i = mid // nblocks2
    g, t = np.meshgrid(np.arange(nblocks2), np.arange(q2i), indexing="ij")
    return _perm_matrix((g * q2i + t).ravel(), (t * nblocks2 + g).ravel(), mid, sparse)


def output_permutation(out: int, nblocks2: int, sparse: bool = False):
    """Q_out with (Q_out v)[p*nblocks2 + g] = v[g*q2o + p]: the inverse stride
    permutation that returns stage 2's block-major result to feature order."""
    q2o = out // nblocks2
    g, p = np.meshgrid(np.arange(nblocks2), np.arange(q2o), indexing="ij")
    return _perm_matrix((p * nblocks2 + g).ravel(), (g * q2o + p).ravel(), out, sparse)


def dense_factors(w1: np.ndarray, w2: np.ndarray, in_features: int, out_features: int,
                  sparse: bool = False):
    """(Rd, Pm, Ld, Qo): the four factor matrices of M = Qo·Ld·Pm·Rd."""
    nb1, nb2 = w1.shape[0], w2.shape[0]
    s = derive_sizes(in_features, out_features, nb1, nb2)
    if w1.shape != (nb1, s["q1o"], s["q1i"]) or w2.shape != (nb2, s["q2o"], s["q2i"]):
        raise ValueError("factor shapes do not match the sizes")
    Rd = block_diag_dense(w1, sparse)
    Pm = stride_permutation(s["mid"], nb2, sparse)
    Ld = block_diag_dense(w2, sparse)
    Qo = output_permutation(s["out"], nb2, sparse)
    return Rd, Pm, Ld, Qo


def monarch_matrix(w1: np.ndarray, w2: np.ndarray, in_features: int, out_features: int) -> np.ndarray:
    """The dense Monarch matrix M = Qo·Ld·Pm·Rd (out x in), fp64."""
    Rd, Pm, Ld, Qo = dense_factors(w1, w2, in_features, out_features)
    return Qo @ (Ld @ (Pm @ Rd))


# ----------------------------------------------------------------------------
# forward and backward
# ----------------------------------------------------------------------------

def _mm(A, B):
    """A @ B where either side may be a scipy sparse matrix; dense result."""
    r = A @ B
    return np.asarray(r.todense()) if hasattr(r, "todense") else np.asarray(r)


def forward(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, in_features: int, out_features: int,
            relu: bool = False, factors=None, keep: bool = False):
    """Y = X·Mᵀ evaluated as X·Rdᵀ·Pmᵀ·Ldᵀ·Qoᵀ with dense factor matrices
    (fp64). relu=True applies max(·, 0) to the result (the ReLU between the
    two layers of the recommender MLP of the "efficiency testing numbers"
    thread). keep=True also returns the intermediates."""
    X = np.asarray(x, dtype=np.float64)
    Rd, Pm, Ld, Qo = factors if factors is not None else dense_factors(w1, w2, in_features, out_features)
    Z = _mm(Rd, X.T).T          # stage 1: block-diagonal R on each row
    W = _mm(Pm, Z.T).T          # stride permutation
    V = _mm(Ld, W.T).T          # stage 2: block-diagonal L
    Y = _mm(Qo, V.T).T          # inverse stride permutation
    if relu:
        Y = np.maximum(Y, 0.0)
    if keep:
        return Y, dict(Z=Z, W=W, V=V)
    return Y


def backward(dy: np.ndarray, x: np.ndarray, w1: np.ndarray, w2: np.ndarray, in_features: int,
             out_features: int, relu: bool = False, y: Optional[np.ndarray] = None, factors=None):
    """Gradients of sum(dY * Y) with respect to X, w1 (R blocks) and w2 (L blocks).

    Chain rule through Y = Qo·Ld·Pm·Rd·x per row (fp64):
        dV = dY_eff·Qo,  dW = dV·Ld,  dZ = dW·Pm,  dX = dZ·Rd,
        dL[g] = diagonal block g of dVᵀ·W,   dR[r] = diagonal block r of dZᵀ·X,
    where dY_eff = dY ⊙ 1[Y > 0] after a fused ReLU (derivative 0 at 0) and
    W = X·Rdᵀ·Pmᵀ is stage 2's input. Returns (dX, dw1, dw2)."""
    X = np.asarray(x, dtype=np.float64)
    dY = np.asarray(dy, dtype=np.float64)
    fac = factors if factors is not None else dense_factors(w1, w2, in_features, out_features)
    Rd, Pm, Ld, Qo = fac
    nb1, nb2 = w1.shape[0], w2.shape[0]
    s = derive_sizes(in_features, out_features, nb1, nb2)
    if relu:
        if y is None:
            y = forward(X, w1, w2, in_features, out_features, relu=True, factors=fac)
        dY = dY * (np.asarray(y, dtype=np.float64) > 0)
    Z = _mm(Rd, X.T).T
    W = _mm(Pm, Z.T).T
    dV = _mm(dY, Qo)
    dW = _mm(dV, Ld)
    dZ = _mm(dW, Pm)
    dX = _mm(dZ, Rd)
    q1o, q1i, q2o, q2i = s["q1o"], s["q1i"], s["q2o"], s["q2i"]
    dw2 = np.empty((nb2, q2o, q2i))
    for g in range(nb2):
        dw2[g] = dV[:, g * q2o:(g + 1) * q2o].T @ W[:, g * q2i:(g + 1) * q2i]
    dw1 = np.empty((nb1, q1o, q1i))
    for r in range(nb1):
        dw1[r] = dZ[:, r * q1o:(r + 1) * q1o].T @ X[:, r * q1i:(r + 1) * q1i]
    return dX, dw1, dw2


def mlp_forward(x, layers: Sequence[Tuple[np.ndarray, np.ndarray, int, int, bool]]):
    """Chain of Monarch layers; each entry is (w1, w2, in, out, relu_after).
    Returns the output and the per-layer inputs/outputs."""
    h = np.asarray(x, dtype=np.float64)
    acts = [h]
    for (w1, w2, fi, fo, relu) in layers:
        h = forward(h, w1, w2, fi, fo, relu=relu)
        acts.append(h)
    return h, acts


def mlp_backward(dy, x, layers):
    """Backward through mlp_forward's chain. Returns (dX, [(dw1, dw2) per layer])."""
    _, acts = mlp_forward(x, layers)
    g = np.asarray(dy, dtype=np.float64)
    grads = [None] * len(layers)
    for i in range(len(layers) - 1, -1, -1):
        w1, w2, fi, fo, relu = layers[i]
        g, dw1, dw2 = backward(g, acts[i], w1, w2, fi, fo, relu=relu, y=acts[i + 1] if relu else None)
        grads[i] = (dw1, dw2)
    return g, grads


# ----------------------------------------------------------------------------
# sampled entries at full size (each output computed on its own)
# ----------------------------------------------------------------------------

def forward_rows(x_rows, w1, w2, in_features, out_features, relu=False, factors=None):
    """Full output rows for a subset of input rows (rows are independent)."""
    return forward(x_rows, w1, w2, in_features, out_features, relu=relu, factors=factors)


def backward_dx_rows(dy_rows, w1, w2, in_features, out_features, factors=None, y_rows=None,
                     relu=False):
    """dX for a subset of rows: dX[b] = dY_eff[b]·Qo·Ld·Pm·Rd."""
    Rd, Pm, Ld, Qo = factors if factors is not None else dense_factors(w1, w2, in_features, out_features)
    dY = np.asarray(dy_rows, dtype=np.float64)
    if relu:
        dY = dY * (np.asarray(y_rows, dtype=np.float64) > 0)
    return _mm(_mm(_mm(_mm(dY, Qo), Ld), Pm), Rd)


def weight_grad_entries(dy, x, w1, w2, in_features, out_features, r_k_s, g_p_t, factors=None,
                        y=None, relu=False, chunk: int = 8192):
    """Individual weight-gradient entries summed over the whole batch.

    dR[r,k,s] = Σ_b dZ[b, r*q1o+k]·X[b, r*q1i+s] with the column dZ[:, j] =
    dY_eff·(Qo·Ld·Pm)[:, j];  dL[g,p,t] = Σ_b dV[b, g*q2o+p]·W[b, g*q2i+t] with
    dV[:, i] = dY_eff·Qo[:, i] and W[:, i] = X·(Pm·Rd)[i, :]ᵀ.
    The batch sum runs over row chunks (fp64) so full-size inputs stay in
    their storage precision in memory."""
    Rd, Pm, Ld, Qo = factors if factors is not None else dense_factors(w1, w2, in_features, out_features)
    s = derive_sizes(in_features, out_features, w1.shape[0], w2.shape[0])
    mid, out = s["mid"], s["out"]
    rcols, rx = [], []
    for (r, k, sidx) in r_k_s:
        e = np.zeros((mid, 1))
        e[r * s["q1o"] + k, 0] = 1.0
        rcols.append(_mm(Qo, _mm(Ld, _mm(Pm, e))).ravel())     # (Qo·Ld·Pm)[:, j]
        rx.append(r * s["q1i"] + sidx)
    lq, lw = [], []
    for (g, p, t) in g_p_t:
        e = np.zeros((out, 1))
        e[g * s["q2o"] + p, 0] = 1.0
        lq.append(_mm(Qo, e).ravel())                          # Qo[:, i_out]
        e2 = np.zeros((1, mid))
        e2[0, g * s["q2i"] + t] = 1.0
        lw.append(_mm(_mm(e2, Pm), Rd).ravel())                # (Pm·Rd)[i_mid, :]
    acc_r = np.zeros(len(rcols))
    acc_l = np.zeros(len(lq))
    nrows = np.asarray(x).shape[0]
    for b0 in range(0, nrows, chunk):
        b1 = min(nrows, b0 + chunk)
        dYc = np.asarray(dy[b0:b1], dtype=np.float64)
        if relu:
            dYc = dYc * (np.asarray(y[b0:b1], dtype=np.float64) > 0)
        Xc = np.asarray(x[b0:b1], dtype=np.float64)
        for i, (col, xi) in enumerate(zip(rcols, rx)):
            acc_r[i] += (dYc @ col) @ Xc[:, xi]
        for i, (qc, wr) in enumerate(zip(lq, lw)):
            acc_l[i] += (dYc @ qc) @ (Xc @ wr)
    return acc_r, acc_l


# ----------------------------------------------------------------------------
# comparison metric
# ----------------------------------------------------------------------------

def rel_frobenius(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_F / ||ref||_F in fp64 (0/0 is 0)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((a - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def max_row_rel_error(a: np.ndarray, ref: np.ndarray, scale: Optional[np.ndarray] = None,
                      floor: float = 1e-3) -> float:
    """Largest relative error of one row, rows taken along the last axis
    (batch rows of activations, block rows of weight gradients).

    With `scale` (the same result computed from the absolute values of every
    input, so each entry is the sum of the magnitudes of the terms it adds
    up), row r is measured as ||a_r - ref_r|| / ||scale_r||: the standard
    bound on the rounding error of a sum is proportional to the magnitudes
    summed, and a row whose terms cancel is then not held to a bound relative
    to its small result. Without cancellation scale_r = |ref_r| and this is
    the plain row-relative error. Without `scale`, row r is measured against
    ||ref_r||, or `floor` times the RMS row norm when that is larger."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    last = ref.shape[-1] if ref.ndim else 1
    a2, r2 = a.reshape(-1, last), ref.reshape(-1, last)
    num = np.linalg.norm(a2 - r2, axis=1)
    if scale is not None:
        den = np.linalg.norm(np.asarray(scale, dtype=np.float64).reshape(-1, last), axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            e = np.where(num == 0.0, 0.0, num / den)
        return float(np.max(e))
    den = np.linalg.norm(r2, axis=1)
    rms = np.linalg.norm(r2) / np.sqrt(r2.shape[0])
    if rms == 0.0:
        return 0.0 if not num.any() else float("inf")
    return float(np.max(num / np.maximum(den, floor * rms)))


def parity_error(a: np.ndarray, ref: np.ndarray, scale: Optional[np.ndarray] = None) -> float:
    """The larger of the whole-tensor relative Frobenius error and the worst
    row's error (max_row_rel_error, against `scale` when given): a result
    passes a bound only if the tensor as a whole and every row of it do."""
    return max(rel_frobenius(a, ref), max_row_rel_error(a, ref, scale))
