"""Float32 quotients a / d that are hardest to round, and matrices whose
factorizations form them, for the check that the kernels' multipliers are
the IEEE float32 quotients bit for bit ("ruSOLVER：小矩阵 kernel 优化
（实验性）", section on the unchanged numerical and failure contract: exact
quotients, no reciprocal approximation).

Write a = A 2^ea, d = D 2^ed with integer significands A, D < 2^24.  In the
normal range a float32 rounding midpoint is m = M 2^em with M odd between
2^24 and 2^25, and A / D = m 2^(ed - ea) would need A = D M 2^k: impossible.
So a normal quotient is never a midpoint, and |A 2^25 - D M| >= 1 bounds
its distance from one; pairs with |A 2^25 - D M| = 1 are the hardest to
round (the exclusion of quotients from midpoints; Muller et al., "Handbook
of Floating-Point Arithmetic", division chapter).  Any shortcut that is
not the correctly rounded division (a reciprocal, a double rounding through
float64 that is off by more than 2^-49 relative) shows on them.  In the
subnormal range the grid is fixed (spacing 2^-149) and exact midpoints
exist: a = D M 2^-149, d = 2 D (D, M odd) gives a / d = M 2^-150, where
ties-to-even decides.

Generators (numpy ``default_rng``; nothing here divides in float32):

  hardest_normal  pairs at the minimal distance from a midpoint,
                  |A 2^25 - D M| = 1 with D odd, A / D in [1/2, 1) (LU
                  multipliers: |a| <= |d|), then scaled by powers of two.
  subnormal_midpoints  exact subnormal midpoints (above).
  underflow       quotients below the normal range, rounding to a
                  subnormal or to zero.
  random_bits     random finite float32 bit patterns of every exponent.
  lu_column_matrix, chol_column_matrix  matrices whose step k0 divides a
                  column of such numerators by one divisor.
"""
from __future__ import annotations

import numpy as np


def f32_bits(u) -> np.ndarray:
    return np.asarray(u, np.uint32).view(np.float32)


def hardest_normal(rng: np.random.Generator, count: int, min_scale: int = 0,
                   max_scale: int = 20, d_exp: int = 0):
    """(a, d) float32 arrays: d = D 2^(d_exp - 23) in [2^d_exp, 2^(d_exp+1)),
    a = A 2^(d_exp - 23 - s) with A / D in [1/2, 1) at distance 1 / (D 2^25)
    from a float32 midpoint, s in [min_scale, max_scale]."""
    out_a, out_d = [], []
    while len(out_a) < count:
        D = int(rng.integers(2 ** 23, 2 ** 24)) | 1
        inv = pow(2 ** 25, -1, D)                 # 2^25 * inv = 1 (mod D)
        for sgn in (1, -1):
            A = (sgn * inv) % D                  # A 2^25 = sgn (mod D)
            if not D // 2 <= A < D:
                continue
            M = (A * 2 ** 25 - sgn) // D
            assert M % 2 == 1 and A * 2 ** 25 - D * M == sgn
            s = int(rng.integers(min_scale, max_scale + 1))
            sa = 1.0 if rng.random() < 0.5 else -1.0
            sd = 1.0 if rng.random() < 0.5 else -1.0
            out_a.append(sa * np.ldexp(float(A), d_exp - 23 - s))
            out_d.append(sd * np.ldexp(float(D), d_exp - 23))
    return (np.array(out_a[:count], np.float32), np.array(out_d[:count], np.float32))


def subnormal_midpoints(rng: np.random.Generator, count: int):
    """(a, d): a = D M 2^-149 (subnormal), d = 2 D, so a / d = M 2^-150, an
    exact midpoint of the subnormal grid (D, M odd, D M < 2^23)."""
    out_a, out_d = [], []
    while len(out_a) < count:
        D = int(rng.integers(1, 2 ** 11)) | 1
        M = int(rng.integers(1, (2 ** 23) // D)) | 1
        if D * M >= 2 ** 23:
            continue
        out_a.append(np.ldexp(float(D * M), -149))
        out_d.append(2.0 * D)
    return np.array(out_a, np.float32), np.array(out_d, np.float32)


def underflow(rng: np.random.Generator, count: int):
    """(a, d) with |a / d| below 2^-126: subnormal quotients and quotients
    that round to zero (|a| <= |d|)."""
    a = np.ldexp(rng.uniform(1.0, 2.0, count), rng.integers(-149, -120, count))
    d = np.ldexp(rng.uniform(1.0, 2.0, count), rng.integers(7, 37, count))
    a = np.where(rng.random(count) < 0.5, -a, a)
    return a.astype(np.float32), d.astype(np.float32)


def random_bits(rng: np.random.Generator, count: int):
    """Random finite float32 operands of every exponent (d non-zero)."""
    a = f32_bits(rng.integers(0, 2 ** 32, count, dtype=np.uint64))
    d = f32_bits(rng.integers(0, 2 ** 32, count, dtype=np.uint64))
    ok = np.isfinite(a) & np.isfinite(d) & (d != 0)
    return a[ok], d[ok]


# ------------------------------------------------- matrices for the kernels


def hardest_numerators(rng: np.random.Generator, count: int, need_sqrt: bool = False):
    """(d, a[count]): a divisor d in [1, 2) and numerators |a| < |d| whose
    quotients a / d sit at the minimal distance from a float32 midpoint
    (the two residues of one odd significand D, scaled by powers of two and
    signed).  need_sqrt: d is also the float32 square root of a float32
    number s (returned third), for the Cholesky kernel."""
    while True:
        D = int(rng.integers(2 ** 23, 2 ** 24)) | 1
        inv = pow(2 ** 25, -1, D)
        As = [A for A in ((inv % D), (-inv) % D) if D // 2 <= A < D]
        if not As:
            continue
        d = np.float32(np.ldexp(float(D), -23))
        s = np.float32(d * d)
        if need_sqrt and np.sqrt(s) != d:
            continue
        a = []
        for i in range(count):
            A = As[i % len(As)]
            v = np.ldexp(float(A), -23 - (i // (2 * len(As))) % 24)
            a.append(-v if (i // len(As)) % 2 else v)
        return d, np.array(a, np.float32), s


def _numerators(rng: np.random.Generator, kind: str, count: int, need_sqrt: bool):
    """(d, a, s) for one column: kinds 'hardest', 'submid' (exact subnormal
    midpoint quotients among ordinary ones), 'underflow', 'random'."""
    if kind == "hardest":
        return hardest_numerators(rng, count, need_sqrt)
    if kind == "submid":
        Dp = int(rng.integers(1, 2 ** 5)) | 1
        d = np.float32(2 * Dp)
        a = []
        for i in range(count):
            if i % 3 == 2:
                a.append(rng.uniform(-1, 1) * Dp)          # an ordinary quotient
            else:
                M = int(rng.integers(1, 2 ** 15)) | 1
                a.append(np.ldexp(float(Dp * M), -149) * (-1 if i % 2 else 1))
        return d, np.array(a, np.float32), np.float32(d * d)
    if kind == "underflow":
        d = np.float32(np.ldexp(rng.uniform(1, 2), 40))
        a = np.ldexp(rng.uniform(1, 2, count), rng.integers(-130, -80, count))
        a[::4] = 0.0
        return d, a.astype(np.float32), np.float32(d * d)
    d = np.float32(4.0)
    return d, rng.uniform(-3.99, 3.99, count).astype(np.float32), np.float32(16.0)


def lu_column_matrix(rng: np.random.Generator, n: int, k0: int, kind: str) -> np.ndarray:
    """Logical float32 n x n matrix: the identity except column k0, which has
    d on the diagonal and numerators below it (|a| < |d|), so steps before k0
    and after take unit pivots with zero multipliers, and step k0 keeps row k0
    as its pivot and forms the multipliers a_i / d of every row below."""
    d, a, _ = _numerators(rng, kind, n - 1 - k0, False)
    A = np.eye(n, dtype=np.float32)
    A[k0, k0] = d
    A[k0 + 1:, k0] = a
    return A


def chol_column_matrix(rng: np.random.Generator, n: int, j0: int, kind: str) -> np.ndarray:
    """Logical float32 symmetric positive definite matrix: the identity on
    the first j0 rows and columns, then s = d^2 (sqrt(s) = d in float32) at
    (j0, j0), the numerators below and right of it, and n s on the rest of
    the diagonal, so step j0 forms the quotients a_i / d."""
    d, a, s = _numerators(rng, kind, n - 1 - j0, kind == "hardest")
    A = np.eye(n, dtype=np.float32)
    A[j0, j0] = s
    A[j0 + 1:, j0] = a
    A[j0, j0 + 1:] = a
    idx = np.arange(j0 + 1, n)
    A[idx, idx] = np.float32(n) * s + np.float32(1.0)
    return A
