"""Accuracy measures used by the tests (not part of the solver).

Norm choices: infinity norms per right-hand-side column, maximum over the
columns of a system.

  normwise error   ||x - x_ref||_inf / ||x_ref||_inf
  residual ratio   ||A x - b||_inf / (n * eps * ||A||_inf * ||x||_inf)
                   evaluated in extended precision from the working-precision
                   A, b and x, eps = unit roundoff of the working type
                   (2**-24 for float32, 2**-53 for float64) times 2, i.e.
                   machine epsilon 2**-23 / 2**-52.
  kappa_inf        ||A||_inf * ||A^-1||_inf in float64.
"""
from __future__ import annotations

import numpy as np

EPS = {np.dtype(np.float32): 2.0 ** -23, np.dtype(np.float64): 2.0 ** -52}
UNIT_ROUNDOFF = {np.dtype(np.float32): 2.0 ** -24, np.dtype(np.float64): 2.0 ** -53}


def normwise_error(X: np.ndarray, Xref: np.ndarray) -> np.ndarray:
    """X, Xref logical [batch, n, nrhs]; returns [batch]."""
    X = np.asarray(X, dtype=np.float64)
    Xref = np.asarray(Xref, dtype=np.float64)
    num = np.abs(X - Xref).max(axis=1)            # [batch, nrhs]
    den = np.abs(Xref).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(den > 0, num / den, np.where(num > 0, np.inf, 0.0))
    return r.max(axis=1)


def residual_ratio(A: np.ndarray, X: np.ndarray, B: np.ndarray, dtype) -> np.ndarray:
    """A logical [batch, n, n], X and B logical [batch, n, nrhs]; returns [batch].

    The product A x is formed in numpy's long double (x87 extended, 64-bit
    significand on x86-64), so its own rounding is far below the float64
    residuals being measured."""
    eps = EPS[np.dtype(dtype)]
    n = A.shape[-1]
    Al = np.asarray(A).astype(np.longdouble)
    Xl = np.asarray(X).astype(np.longdouble)
    Bl = np.asarray(B).astype(np.longdouble)
    R = np.matmul(Al, Xl) - Bl                    # [batch, n, nrhs]
    rnorm = np.abs(R).max(axis=1).astype(np.float64)          # [batch, nrhs]
    anorm = np.abs(np.asarray(A, dtype=np.float64)).sum(axis=2).max(axis=1)  # [batch]
    xnorm = np.abs(np.asarray(X, dtype=np.float64)).max(axis=1)               # [batch, nrhs]
    den = n * eps * anorm[:, None] * xnorm
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(den > 0, rnorm / den, np.where(rnorm > 0, np.inf, 0.0))
    return r.max(axis=1)


def kappa_inf(A: np.ndarray) -> np.ndarray:
    """Condition number in the infinity norm, float64; inf where singular.
    Batched: numpy's cond inverts the whole stack at once and turns the NaN
    of an exactly singular matrix into inf."""
    A = np.asarray(A, dtype=np.float64)
    if A.shape[0] == 0:
        return np.zeros(0)
    return np.asarray(np.linalg.cond(A, p=np.inf), dtype=np.float64).reshape(A.shape[0])


def apply_swaps(M: np.ndarray, ipiv: np.ndarray) -> np.ndarray:
    """Apply a 0-based LAPACK swap sequence to the rows of each matrix:
    for k in order, rows k and ipiv[k] are exchanged.  M [batch, n, m]."""
    out = np.array(M, copy=True)
    for s in range(out.shape[0]):
        for k, p in enumerate(ipiv[s]):
            if p != k:
                out[s, [k, p]] = out[s, [p, k]]
    return out
