"""Pins of the CPU oracle against facts fixed outside it.

Each test ties the oracle to something it cannot reproduce by itself being
wrong in the same way: hand-worked examples, exact rational arithmetic
(Cramer's rule, exact Gaussian elimination), the textbook backward-error
bound of LU factorization, LAPACK's pivot sequence, closed forms of special
matrices and exact-singularity constructions.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import golden_io
import metrics
import oracle

DTYPES = [np.float64, np.float32]
LAYOUTS = ["row", "col"]


def _solve_logical(A, B, dtype, layout, nthreads=0):
    """Run the oracle on logical A [batch,n,n], B [batch,n,nrhs]."""
    A = np.asarray(A, dtype=dtype)
    B = np.asarray(B, dtype=dtype)
    n, nrhs = A.shape[1], B.shape[2]
    X_st, piv, info = oracle.gesv(oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout),
                                  n, nrhs, layout, nthreads)
    return oracle.rhs_from_storage(X_st, layout, n, nrhs), piv, info


def _factor_logical(A, dtype, layout):
    A = np.asarray(A, dtype=dtype)
    return oracle.getrf(oracle.to_storage(A, layout), A.shape[1], layout)


# ---------------------------------------------------------------- hand-worked


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("embed", [None, 8])
def test_golden_examples(dtype, layout, embed):
    for ex in golden_io.all_examples():
        if embed:
            ex = golden_io.embed_identity(ex, embed)
        A = ex["A"][None]
        b = ex["b"][None, :, None]
        X, piv, info = _solve_logical(A, b, dtype, layout)
        assert info[0] == ex["info"], ex["name"]
        np.testing.assert_array_equal(piv[0], ex["piv"], err_msg=ex["name"])
        # every value of these examples is a dyadic rational: exact equality
        np.testing.assert_array_equal(X[0, :, 0], ex["x"].astype(dtype), err_msg=ex["name"])
        if ex["info"] != 0:
            assert not np.signbit(X).any(), "failed system must hold +0.0"
        LU, ipiv, ginfo, _ = _factor_logical(A, dtype, layout)
        np.testing.assert_array_equal(ipiv[0], ex["ipiv"], err_msg=ex["name"])
        assert ginfo[0] == ex["getrf_info"]
        if "L" in ex:
            L = np.tril(LU[0], -1) + np.eye(3)
            U = np.triu(LU[0])
            np.testing.assert_array_equal(L, ex["L"].astype(dtype))
            np.testing.assert_array_equal(U, ex["U"].astype(dtype))


# ------------------------------------------------------ exact rational pins


def _det(M):
    """Exact determinant by cofactor expansion (n <= 4)."""
    n = len(M)
    if n == 1:
        return M[0][0]
    if n == 2:
        return M[0][0] * M[1][1] - M[0][1] * M[1][0]
    total = Fraction(0)
    for c in range(n):
        minor = [row[:c] + row[c + 1:] for row in M[1:]]
        total += (-1) ** c * M[0][c] * _det(minor)
    return total


def _cramer(A, b):
    n = len(A)
    M = [[Fraction(float(v)) for v in row] for row in A]
    bb = [Fraction(float(v)) for v in b]
    d = _det(M)
    if d == 0:
        return None
    x = []
    for i in range(n):
        Mi = [row[:i] + [bb[r]] + row[i + 1:] for r, row in enumerate(M)]
        x.append(_det(Mi) / d)
    return x


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_cramer_exact(dtype, layout, n):
    """Solution vs Cramer's rule in exact rationals from the exact inputs.

    Bound: the computed x solves (A + dA) x = b with |dA| <= gamma_3n |L||U|
    (backward error of Gaussian elimination), |L||U| <= n * 2**(n-1) |A| in
    norm under partial pivoting, so the forward error is at most
    kappa * gamma_3n * n * 2**(n-1) / (1 - that)."""
    rng = np.random.default_rng(100 + n)
    batch = 300
    A = rng.uniform(-1, 1, size=(batch, n, n)).astype(dtype)
    B = rng.uniform(-1, 1, size=(batch, n, 2)).astype(dtype)
    X, piv, info = _solve_logical(A, B, dtype, layout)
    u = metrics.UNIT_ROUNDOFF[np.dtype(dtype)]
    kappa = metrics.kappa_inf(A.astype(np.float64))
    gamma = 3 * n * u / (1 - 3 * n * u)
    checked = 0
    for s in range(batch):
        if not np.isfinite(kappa[s]) or kappa[s] > 1e6:
            continue
        assert info[s] == 0
        f = kappa[s] * gamma * n * 2 ** (n - 1)
        bound = f / (1 - f)
        for j in range(2):
            xs = _cramer(A[s], B[s, :, j])
            xs_f = np.array([float(v) for v in xs])
            err = np.abs(X[s, :, j].astype(np.float64) - xs_f).max() / np.abs(xs_f).max()
            assert err <= bound, (s, j, err, bound)
        checked += 1
    assert checked > batch // 2


def _exact_gepp(A):
    """Gaussian elimination with partial pivoting in exact rationals, first
    maximum in increasing current position.  Returns (ipiv, singular_step)."""
    n = len(A)
    M = [[Fraction(float(v)) for v in row] for row in A]
    ipiv = []
    first_zero = 0
    for k in range(n):
        p = k
        for r in range(k + 1, n):
            if abs(M[r][k]) > abs(M[p][k]):
                p = r
        ipiv.append(p)
        if M[p][k] == 0:
            if first_zero == 0:
                first_zero = k + 1
            continue
        M[k], M[p] = M[p], M[k]
        for r in range(k + 1, n):
            l = M[r][k] / M[k][k]
            for c in range(k, n):
                M[r][c] -= l * M[k][c]
    return ipiv, first_zero


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [2, 3, 5, 6])
def test_exact_gepp_pivots(dtype, n):
    """Pivot sequence vs exact-rational elimination on inputs whose float
    pivot gap is comfortable (rounding cannot flip the choice there)."""
    rng = np.random.default_rng(7 + n)
    A = rng.uniform(-1, 1, size=(200, n, n)).astype(dtype)
    _, ipiv, info, gap = _factor_logical(A, dtype, "row")
    checked = 0
    for s in range(A.shape[0]):
        if gap[s] < 1e-3:
            continue
        ex_piv, ex_zero = _exact_gepp(A[s])
        np.testing.assert_array_equal(ipiv[s], ex_piv)
        assert info[s] == ex_zero
        checked += 1
    assert checked > 100


def test_exact_gepp_integer_ties():
    """Small-integer matrices have many exact magnitude ties; whenever every
    float step is exact (checked by comparing against the rational run),
    the tie decisions must agree with exact elimination."""
    rng = np.random.default_rng(3)
    agree = 0
    for _ in range(400):
        n = int(rng.integers(2, 6))
        A = rng.integers(-2, 3, size=(n, n)).astype(np.float64)
        ex_piv, ex_zero = _exact_gepp(A)
        LU, ipiv, info, _ = _factor_logical(A[None], np.float64, "row")
        if ex_zero == 0 and np.isfinite(LU).all():
            # exact rational factors, rounded: if they are representable the
            # float run followed the exact one step by step
            P = metrics.apply_swaps(A[None], np.array([ex_piv]))[0]
            L = np.tril(LU[0], -1) + np.eye(n)
            U = np.triu(LU[0])
            if np.array_equal(L @ U, P):
                np.testing.assert_array_equal(ipiv[0], ex_piv)
                agree += 1
    assert agree > 100


# ----------------------------------------------------- factorization bound


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_reconstruction_bound(dtype, layout):
    """|P A - L U| <= gamma_n |L| |U| componentwise (backward error of the
    computed LU factors), and |L_ij| <= 1 (partial pivoting), for random n in
    [1, 64] and several value distributions."""
    rng = np.random.default_rng(11)
    u = metrics.UNIT_ROUNDOFF[np.dtype(dtype)]
    for trial in range(40):
        n = int(rng.integers(1, 65))
        kind = trial % 4
        if kind == 0:
            A = rng.uniform(-1, 1, size=(3, n, n))
        elif kind == 1:
            A = rng.standard_normal(size=(3, n, n)) + 0.5 * np.eye(n)
        elif kind == 2:
            A = rng.uniform(-1, 1, size=(3, n, n)) * 10.0 ** rng.uniform(-3, 3, size=(3, n, 1))
        else:
            A = rng.standard_normal(size=(3, n, n)) * 10.0 ** rng.uniform(-3, 3, size=(3, 1, n))
        A = A.astype(dtype)
        LU, ipiv, info, _ = _factor_logical(A, dtype, layout)
        gamma = n * u / (1 - n * u)
        for s in range(A.shape[0]):
            L = (np.tril(LU[s], -1) + np.eye(n)).astype(np.longdouble)
            U = np.triu(LU[s]).astype(np.longdouble)
            PA = metrics.apply_swaps(A[s][None].astype(np.longdouble), ipiv[s][None])[0]
            diff = np.abs(PA - L @ U)
            bound = gamma * (np.abs(L) @ np.abs(U))
            # the extended-precision product adds at most n * 2**-64 relative
            slack = n * 2.0 ** -63 * (np.abs(L) @ np.abs(U))
            assert (diff <= bound + slack).all(), (n, trial, s)
            assert (np.abs(np.tril(LU[s], -1)) <= 1).all()


# ------------------------------------------------------------ LAPACK pivots


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_lapack_pivots(dtype, layout):
    """ipiv equals LAPACK getrf's (scipy lu_factor, 0-based) on inputs whose
    pivot gap leaves no room for rounding to flip a choice; U agrees within
    rounding; the solution agrees with LAPACK gesv within kappa-scaled bounds."""
    rng = np.random.default_rng(5)
    thr = 1e-9 if dtype == np.float64 else 1e-4
    u = metrics.UNIT_ROUNDOFF[np.dtype(dtype)]
    checked = 0
    for trial in range(60):
        n = int(rng.integers(1, 65))
        A = rng.standard_normal(size=(4, n, n)).astype(dtype)
        B = rng.standard_normal(size=(4, n, 3)).astype(dtype)
        LU, ipiv, info, gap = _factor_logical(A, dtype, layout)
        X, piv, sinfo = _solve_logical(A, B, dtype, layout)
        for s in range(A.shape[0]):
            if gap[s] < thr:
                continue
            lu, lpiv = scipy.linalg.lu_factor(A[s], check_finite=False)
            np.testing.assert_array_equal(ipiv[s], lpiv.astype(np.int32))
            np.testing.assert_array_equal(piv[s], lpiv.astype(np.int32))
            assert info[s] == 0 and sinfo[s] == 0
            scale = np.abs(np.triu(lu)).max()
            assert np.abs(np.triu(LU[s]) - np.triu(lu)).max() <= 64 * n * u * scale * 10
            xl = scipy.linalg.lu_solve((lu, lpiv), B[s], check_finite=False)
            kap = metrics.kappa_inf(A[s][None].astype(np.float64))[0]
            err = np.abs(X[s] - xl).max() / np.abs(xl).max()
            assert err <= 8 * n * n * u * kap + 1e-300, (n, err)
            checked += 1
    assert checked > 150


# ---------------------------------------------------------- special cases


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_special_matrices(dtype, layout):
    rng = np.random.default_rng(21)
    for n in (1, 2, 7, 8, 16, 24, 33, 64):
        nrhs = 3
        B = rng.uniform(-1, 1, size=(1, n, nrhs)).astype(dtype)
        # identity: x = b, no swaps
        X, piv, info = _solve_logical(np.eye(n)[None], B, dtype, layout)
        np.testing.assert_array_equal(X, B)
        np.testing.assert_array_equal(piv[0], np.arange(n))
        assert info[0] == 0
        # permutation matrix P (A[i, perm[i]] = 1): x[perm[i]] = b[i], exactly
        perm = rng.permutation(n)
        P = np.zeros((n, n))
        P[np.arange(n), perm] = 1
        X, piv, info = _solve_logical(P[None], B, dtype, layout)
        expect = np.empty_like(B[0])
        expect[perm] = B[0]
        np.testing.assert_array_equal(X[0], expect)
        assert info[0] == 0
        # diagonal: x = b / d correctly rounded
        d = rng.uniform(0.5, 2.0, size=n) * rng.choice([-1, 1], size=n)
        D = np.diag(d).astype(dtype)
        X, piv, info = _solve_logical(D[None], B, dtype, layout)
        np.testing.assert_array_equal(X[0], B[0] / d.astype(dtype)[:, None])
        np.testing.assert_array_equal(piv[0], np.arange(n))
        # upper triangular with a non-zero diagonal: no swap
        Uu = np.triu(rng.uniform(-1, 1, size=(n, n))) + np.diag(rng.uniform(1, 2, size=n))
        X, piv, info = _solve_logical(Uu[None], B, dtype, layout)
        np.testing.assert_array_equal(piv[0], np.arange(n))
        assert info[0] == 0
        # x = U^-1 b by the same back substitution order -> scipy agrees closely
        xs = scipy.linalg.solve_triangular(Uu.astype(dtype), B[0])
        assert np.abs(X[0] - xs).max() <= 1e3 * n * metrics.EPS[np.dtype(dtype)] * np.abs(xs).max()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_power_of_two_scaling(dtype, layout):
    """A * 2**j gives the same pivots and x * 2**-j bit for bit (power-of-two
    scaling is exact, so every multiplier is unchanged)."""
    rng = np.random.default_rng(8)
    A = rng.standard_normal(size=(50, 20, 20)).astype(dtype)
    B = rng.standard_normal(size=(50, 20, 2)).astype(dtype)
    X0, piv0, info0 = _solve_logical(A, B, dtype, layout)
    for j in (-7, 3, 11):
        X1, piv1, info1 = _solve_logical(A * dtype(2.0 ** j), B, dtype, layout)
        np.testing.assert_array_equal(piv1, piv0)
        np.testing.assert_array_equal(info1, info0)
        np.testing.assert_array_equal(X1, X0 * dtype(2.0 ** -j))


# ------------------------------------------------------------ singularity


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_exact_singularity_constructions(dtype, layout):
    """Constructions whose first zero pivot is known exactly.

    * two bitwise-equal rows: while neither is the pivot both receive the
      same updates; once one is the pivot the other gets the multiplier 1
      (exact quotient) and becomes exactly zero, a zero row that can only be
      the last pivot -> status n.
    * a zero row -> status n.  * zero column j -> status j+1.
    * zero matrix -> status 1."""
    rng = np.random.default_rng(13)
    for n in (2, 3, 8, 16, 24, 32, 64):
        batch = 40
        A = rng.uniform(-1, 1, size=(batch, n, n)).astype(dtype)
        B = rng.uniform(-1, 1, size=(batch, n, 1)).astype(dtype)
        for s in range(batch):
            i, k = rng.choice(n, size=2, replace=False)
            A[s, k] = A[s, i]
        X, piv, info = _solve_logical(A, B, dtype, layout)
        assert (info == n).all(), (n, info)
        assert (piv == -1).all() and (X == 0).all() and not np.signbit(X).any()
        # zero row
        A = rng.uniform(-1, 1, size=(batch, n, n)).astype(dtype)
        A[np.arange(batch), rng.integers(0, n, size=batch)] = 0
        _, _, info = _solve_logical(A, B, dtype, layout)
        assert (info == n).all()
        # zero column j
        A = rng.uniform(-1, 1, size=(batch, n, n)).astype(dtype)
        cols = rng.integers(0, n, size=batch)
        A[np.arange(batch), :, cols] = 0
        _, _, info = _solve_logical(A, B, dtype, layout)
        np.testing.assert_array_equal(info, cols + 1)
        # zero matrix
        _, piv, info = _solve_logical(np.zeros((1, n, n)), B[:1], dtype, layout)
        assert info[0] == 1 and (piv == -1).all()


# -------------------------------------------------------------- pivot gap


def test_pivot_gap_values():
    """Gap of hand-built columns: first column (4, 3, -1) -> (4-3)/4; later
    steps of an upper-triangular matrix have one non-zero candidate -> 1."""
    A = np.array([[[4.0, 0, 0], [3.0, 1, 0], [-1.0, 0, 1]]])
    _, _, _, gap = oracle.getrf(oracle.to_storage(A, "row"), 3, "row")
    # step 0: (4-3)/4 = 0.25.  step 1: after l = 0.75, -0.25 the column 1
    # candidates are 1 and 0 -> gap 1.
    assert gap[0] == 0.25
    T = np.triu(np.ones((5, 5))) * 2
    _, _, _, gap = oracle.getrf(oracle.to_storage(T[None], "row"), 5, "row")
    assert gap[0] == 1.0
    Z = np.array([[[1.0, 2.0], [-1.0, 5.0]]])
    _, _, _, gap = oracle.getrf(oracle.to_storage(Z, "row"), 2, "row")
    assert gap[0] == 0.0


# ------------------------------------------------------------- layouts


@pytest.mark.parametrize("dtype", DTYPES)
def test_layouts_bitwise_equal(dtype):
    """The layout flag only changes addressing: the same logical system gives
    identical bits in both layouts (and each layout is pinned by the tests
    above against facts about the logical matrix)."""
    rng = np.random.default_rng(17)
    A = rng.standard_normal(size=(64, 24, 24)).astype(dtype)
    B = rng.standard_normal(size=(64, 24, 3)).astype(dtype)
    Xr, pr, ir = _solve_logical(A, B, dtype, "row")
    Xc, pc, ic = _solve_logical(A, B, dtype, "col")
    np.testing.assert_array_equal(Xr, Xc)
    np.testing.assert_array_equal(pr, pc)
    np.testing.assert_array_equal(ir, ic)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(19)
    A = rng.standard_normal(size=(257, 16, 16))
    B = rng.standard_normal(size=(257, 16, 4))
    X1, p1, i1 = _solve_logical(A, B, np.float64, "row", nthreads=1)
    X4, p4, i4 = _solve_logical(A, B, np.float64, "row", nthreads=4)
    np.testing.assert_array_equal(X1, X4)
    np.testing.assert_array_equal(p1, p4)


def test_empty_batch():
    X, piv, info = oracle.gesv(np.zeros((0,)), np.zeros((0,)), 8, 1, "row")
    assert X.size == 0 and piv.shape == (0, 8) and info.shape == (0,)


# ------------------------------------------------------------- getrs (split)


def _random_swaps(rng, n):
    """A LAPACK swap sequence: piv[k] drawn from k..n-1."""
    return np.array([rng.integers(k, n) for k in range(n)], dtype=np.int32)


def _exact_factor_system(rng, n, nrhs):
    """Integer factors with an exactly known solution.

    L unit lower and U upper with small integer entries, U's diagonal in
    {+-1, +-2, +-4}, a random swap sequence piv and an integer solution x;
    b = P^-1 (L U x) formed in exact integer arithmetic.  Every value the
    substitutions meet is then a dyadic rational of a few bits, so a correct
    getrs returns x exactly in float32 and float64."""
    L = np.tril(rng.integers(-2, 3, (n, n)), -1) + np.eye(n, dtype=np.int64)
    U = np.triu(rng.integers(-2, 3, (n, n)), 1)
    U += np.diag(rng.choice([-4, -2, -1, 1, 2, 4], n))
    piv = _random_swaps(rng, n)
    x = rng.integers(-3, 4, (n, nrhs))
    c = L @ (U @ x)                      # = P b
    b = c.copy()
    for k in range(n - 1, -1, -1):       # undo the swaps, last first
        b[[k, piv[k]]] = b[[piv[k], k]]
    LU = np.tril(L, -1) + U
    return LU, piv, b, x


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_getrs_exact_integer_factors(dtype, layout):
    """Solving from hand-made factors gives the exact solution (pins the swap
    order, the unit diagonal of L, and which triangle is read where)."""
    rng = np.random.default_rng(11)
    for n, nrhs in [(1, 1), (3, 2), (6, 1), (9, 4), (16, 3)]:
        LU, piv, b, x = _exact_factor_system(rng, n, nrhs)
        X = oracle.getrs(oracle.to_storage(LU[None].astype(dtype), layout), piv[None],
                         oracle.rhs_to_storage(b[None].astype(dtype), layout), n, nrhs, layout)
        Xl = oracle.rhs_from_storage(X, layout, n, nrhs)[0]
        np.testing.assert_array_equal(Xl, x.astype(dtype), err_msg=f"n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_getrs_matches_lapack(dtype, layout):
    """Against LAPACK's getrs (SciPy lu_solve) on LAPACK's own factors."""
    rng = np.random.default_rng(12)
    n, nrhs, batch = 12, 3, 40
    A = rng.standard_normal((batch, n, n)) + 4 * np.eye(n)
    B = rng.standard_normal((batch, n, nrhs))
    A = A.astype(dtype)
    B = B.astype(dtype)
    tol = 50 * n * np.finfo(dtype).eps
    for s in range(batch):
        lu, piv = scipy.linalg.lu_factor(A[s])
        ref = scipy.linalg.lu_solve((lu, piv), B[s])
        X = oracle.getrs(oracle.to_storage(lu[None], layout), piv[None].astype(np.int32),
                         oracle.rhs_to_storage(B[s][None], layout), n, nrhs, layout)
        Xl = oracle.rhs_from_storage(X, layout, n, nrhs)[0]
        err = np.abs(Xl - ref).max() / np.abs(ref).max()
        assert err <= tol, (s, err)


@pytest.mark.parametrize("dtype", DTYPES)
def test_getrs_failed_factorization_gives_zero(dtype):
    n, nrhs = 5, 2
    LU = np.ones((2, n, n), dtype=dtype)
    piv = np.full((2, n), -1, dtype=np.int32)
    piv[1] = np.arange(n)
    LU[1] = np.eye(n, dtype=dtype)
    B = np.full((2, n, nrhs), -3.0, dtype=dtype)
    X = oracle.getrs(LU, piv, B, n, nrhs, "row")
    assert (X[0] == 0).all() and not np.signbit(X[0]).any()
    np.testing.assert_array_equal(X[1], B[1])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_factor_then_solve_is_gesv(dtype, layout):
    """getrs after getrf repeats gesv's operations in gesv's order: the
    same bits (singular systems included: both give +0.0)."""
    rng = np.random.default_rng(13)
    n, nrhs, batch = 10, 2, 60
    A = rng.uniform(-1, 1, (batch, n, n)).astype(dtype)
    A[::7, 4] = A[::7, 1]                       # some exactly singular systems
    B = rng.uniform(-1, 1, (batch, n, nrhs)).astype(dtype)
    As, Bs = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X, piv, info = oracle.gesv(As, Bs, n, nrhs, layout)
    LU, ipiv, finfo, _ = oracle.getrf(As, n, layout)
    np.testing.assert_array_equal(info, finfo)
    ipiv = np.where(finfo[:, None] != 0, -1, ipiv).astype(np.int32)   # failed: pivots -1
    X2 = oracle.getrs(oracle.to_storage(LU, layout), ipiv, Bs, n, nrhs, layout)
    assert np.array_equal(X.view(np.uint8), X2.view(np.uint8))
    assert (info[::7] != 0).all()


# ---------------------------------------------------------------- Cholesky


def _exact_spd(rng, n, nrhs):
    """L with small integer entries below the diagonal and a diagonal in
    {1, 2, 4}, A = L L^T and b = A x for an integer x, all exact integers:
    the factorization meets perfect squares and exact quotients only, so a
    correct potrf returns L and a correct posv returns x, bit for bit."""
    L = np.tril(rng.integers(-2, 3, (n, n)), -1) + np.diag(rng.choice([1, 2, 4], n))
    A = L @ L.T
    x = rng.integers(-3, 4, (n, nrhs))
    return L, A, x, A @ x


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_cholesky_exact_integer_factors(dtype, layout):
    rng = np.random.default_rng(21)
    for n, nrhs in [(1, 1), (2, 3), (5, 1), (8, 2), (12, 4)]:
        L, A, x, b = _exact_spd(rng, n, nrhs)
        Lo, info = oracle.potrf(oracle.to_storage(A[None].astype(dtype), layout), n, layout)
        assert info[0] == 0
        np.testing.assert_array_equal(Lo[0], L.astype(dtype), err_msg=f"n={n}")
        X, info = oracle.posv(oracle.to_storage(A[None].astype(dtype), layout),
                              oracle.rhs_to_storage(b[None].astype(dtype), layout), n, nrhs,
                              layout)
        np.testing.assert_array_equal(oracle.rhs_from_storage(X, layout, n, nrhs)[0],
                                      x.astype(dtype), err_msg=f"n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_cholesky_matches_lapack(dtype, layout):
    """Against LAPACK's potrf/potrs (SciPy cho_factor / cho_solve)."""
    rng = np.random.default_rng(22)
    n, nrhs, batch = 16, 3, 30
    M = rng.standard_normal((batch, n, n))
    A = (M @ M.transpose(0, 2, 1) + n * np.eye(n)).astype(dtype)
    A = (A + A.transpose(0, 2, 1)) / 2                   # exactly symmetric after rounding
    B = rng.standard_normal((batch, n, nrhs)).astype(dtype)
    L, info = oracle.potrf(oracle.to_storage(A, layout), n, layout)
    X, xinfo = oracle.posv(oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout), n,
                           nrhs, layout)
    X = oracle.rhs_from_storage(X, layout, n, nrhs)
    assert (info == 0).all() and (xinfo == 0).all()
    tol = 50 * n * np.finfo(dtype).eps
    for s in range(batch):
        c, low = scipy.linalg.cho_factor(A[s], lower=True)
        ref_L = np.tril(c)
        assert np.abs(L[s] - ref_L).max() <= tol * np.abs(ref_L).max(), s
        ref_x = scipy.linalg.cho_solve((c, low), B[s])
        assert np.abs(X[s] - ref_x).max() <= tol * np.abs(ref_x).max() * 10, s


def test_cholesky_first_failing_minor():
    """Status j+1 for the smallest leading minor that is not positive
    definite, pinned by the eigenvalues of the leading blocks."""
    rng = np.random.default_rng(23)
    n = 9
    checked = 0
    for _ in range(200):
        Q = np.linalg.qr(rng.standard_normal((n, n)))[0]
        ev = rng.uniform(0.5, 2.0, n)
        ev[rng.integers(0, n)] = -rng.uniform(0.5, 2.0)       # indefinite
        A = Q @ np.diag(ev) @ Q.T
        A = (A + A.T) / 2
        mins = [np.linalg.eigvalsh(A[:k, :k]).min() for k in range(1, n + 1)]
        first = next(k for k, m in enumerate(mins, 1) if m <= 0)
        if min(abs(m) for m in mins) < 1e-6:
            continue                                          # too close to call
        L, info = oracle.potrf(A[None], n, "row")
        assert info[0] == first
        assert (L == 0).all() and not np.signbit(L).any()
        checked += 1
    assert checked > 100


@pytest.mark.parametrize("dtype", DTYPES)
def test_cholesky_symmetry_and_shift(dtype):
    rng = np.random.default_rng(24)
    n = 7
    L0, A, x, b = _exact_spd(rng, n, 1)
    A = A.astype(dtype)
    # one off-diagonal pair differs by one unit in the last place: -2
    Ab = A.copy()
    Ab[5, 2] = np.nextafter(Ab[5, 2], dtype(np.inf))
    L, info = oracle.potrf(np.stack([A, Ab]), n, "row")
    assert list(info) == [0, -2]
    X, xinfo = oracle.posv(np.stack([A, Ab]), np.stack([b, b]).astype(dtype), n, 1, "row")
    assert list(xinfo) == [0, -2] and (X[1] == 0).all() and not np.signbit(X[1]).any()
    # the shift is added to the diagonal once, nothing else: potrf(A, s) is
    # potrf(A + s I) whenever A(j,j) + s is exact
    s = 3.0
    L1, _ = oracle.potrf(A[None], n, "row", shift=s)
    L2, _ = oracle.potrf((A + s * np.eye(n, dtype=dtype))[None], n, "row")
    np.testing.assert_array_equal(L1, L2)
    # a shift that makes the first pivot non-positive fails at step 1
    _, info = oracle.potrf(A[None], n, "row", shift=-float(A[0, 0]))
    assert info[0] == 1


# ------------------------------------------------- non-finite statuses, scaling
#
# ruSOLVER's status codes: -1 for a non-finite input, -3 for a non-finite
# intermediate result, after the positive status of a failed pivot; a failed
# system is zeroed.  The cases below are built by hand so that the status is
# fixed by the arithmetic itself (an exact value beyond the largest finite
# number must round to infinity).

def _fmax(dtype):
    return float(np.finfo(dtype).max)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_nonfinite_input_status(dtype, layout):
    rng = np.random.default_rng(41)
    n, nrhs, batch = 6, 2, 12
    A = rng.uniform(-1, 1, (batch, n, n)).astype(dtype)
    B = rng.uniform(-1, 1, (batch, n, nrhs)).astype(dtype)
    X0, piv0, info0 = _solve_logical(A, B, dtype, layout)
    assert (info0 == 0).all()
    bad = {1: ("A", np.nan), 4: ("A", np.inf), 5: ("B", -np.inf), 9: ("B", np.nan),
           10: ("A", -np.inf)}
    A1, B1 = A.copy(), B.copy()
    for s, (which, v) in bad.items():
        if which == "A":
            A1[s, rng.integers(n), rng.integers(n)] = v
        else:
            B1[s, rng.integers(n), rng.integers(nrhs)] = v
    expect = np.where(~np.isfinite(A1).all(axis=(1, 2)) | ~np.isfinite(B1).all(axis=(1, 2)),
                      -1, 0)
    X, piv, info = _solve_logical(A1, B1, dtype, layout)
    np.testing.assert_array_equal(info, expect)
    for s in range(batch):
        if s in bad:
            assert (X[s] == 0).all() and not np.signbit(X[s]).any() and (piv[s] == -1).all()
        else:   # the other systems are untouched
            np.testing.assert_array_equal(X[s], X0[s])
            np.testing.assert_array_equal(piv[s], piv0[s])
    LU, ipiv, finfo, _ = _factor_logical(A1, dtype, layout)
    np.testing.assert_array_equal(finfo, np.where(~np.isfinite(A1).all(axis=(1, 2)), -1, 0))
    # -1 comes before a zero pivot: a singular matrix with a NaN right-hand side
    Z = np.zeros((1, n, n), dtype)
    Bn = np.full((1, n, 1), np.nan, dtype)
    assert _solve_logical(Z, Bn, dtype, layout)[2][0] == -1


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_overflow_gives_minus3(dtype, layout):
    M = 0.75 * _fmax(dtype)
    # the update -M - 1*M = -1.5 max overflows to -inf in U(1,1)
    A = np.array([[[1, M], [1, -M]]], dtype)
    b = np.array([[[1], [1]]], dtype)
    X, piv, info = _solve_logical(A, b, dtype, layout)
    assert info[0] == -3 and (X == 0).all() and (piv == -1).all()
    assert _factor_logical(A, dtype, layout)[2][0] == -3
    # finite factors, but the solution 2^100 / 2^-1000 (f32: 2^20 / 2^-120)
    # is beyond the range
    e_small, e_big = (-1000, 100) if dtype == np.float64 else (-120, 20)
    A = np.array([[[2.0 ** e_small]]], dtype)
    b = np.array([[[2.0 ** e_big]]], dtype)
    X, piv, info = _solve_logical(A, b, dtype, layout)
    assert info[0] == -3 and X[0, 0, 0] == 0
    assert _factor_logical(A, dtype, layout)[2][0] == 0
    # a zero pivot comes before -3: same overflow, then a zero column
    A = np.array([[[1, M, 0], [1, -M, 0], [0, 0, 0]]], dtype)
    X, piv, info = _solve_logical(A, np.ones((1, 3, 1), dtype), dtype, layout)
    assert info[0] == 3


@pytest.mark.parametrize("dtype", DTYPES)
def test_nan_candidate_ranks_above_zero(dtype):
    # Step 0 (ties to position 0) sends -inf to positions 1 and 3 of column
    # 1; step 1 takes the first (-inf), so position 2 gets the multiplier
    # 1/-inf = -0 and keeps an exact 0 in column 2, while position 3 gets
    # -inf/-inf = NaN.  At step 2 the candidates are 0 (position 2) and NaN
    # (position 3): NaN ranks above, so there is no zero pivot and the
    # non-finite factors give -3.  A search in which NaN never wins would stop
    # at a zero pivot (status 3).
    M = 0.75 * _fmax(dtype)
    A = np.array([[[1, M, 0, 0],
                   [1, -M, 1, 0],
                   [0, 1, 0, 1],
                   [1, -M, 0, 0]]], dtype)
    X, piv, info = _solve_logical(A, np.ones((1, 4, 1), dtype), dtype, "row")
    assert info[0] == -3
    assert _factor_logical(A, dtype, "col")[2][0] == -3


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_scaling_by_power_of_two_is_exact(dtype, layout):
    # When the largest magnitude is a power of two, dividing by it and
    # multiplying U back are exact, so the scaled solve and factorization
    # are bitwise the unscaled ones.
    rng = np.random.default_rng(43)
    n, nrhs, batch = 9, 3, 40
    A = rng.uniform(-1, 1, (batch, n, n))
    e = rng.integers(-6, 7, batch)
    for s in range(batch):
        A[s, rng.integers(n), rng.integers(n)] = rng.choice([-1.0, 1.0])
        A[s] *= 2.0 ** e[s]
    A = A.astype(dtype)
    B = rng.uniform(-1, 1, (batch, n, nrhs)).astype(dtype)
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X0, p0, i0 = oracle.gesv(A_st, B_st, n, nrhs, layout)
    X1, p1, i1 = oracle.gesv(A_st, B_st, n, nrhs, layout, scale=True)
    np.testing.assert_array_equal(X1, X0)
    np.testing.assert_array_equal(p1, p0)
    np.testing.assert_array_equal(i1, i0)
    LU0, q0, f0, _ = oracle.getrf(A_st, n, layout)
    LU1, q1, f1, _ = oracle.getrf(A_st, n, layout, scale=True)
    np.testing.assert_array_equal(LU1, LU0)
    np.testing.assert_array_equal(q1, q0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_scaling_general(dtype):
    # Any scale: the solution is LAPACK's within the working-precision
    # error bound, and the restored factors rebuild P A within the textbook
    # bound.  A large common factor shows that U is restored (its scale is
    # that of A) and that B is scaled with A (else x would be off by it).
    rng = np.random.default_rng(44)
    n, batch = 8, 30
    A = (rng.normal(size=(batch, n, n)) * 37.0).astype(dtype)
    B = rng.normal(size=(batch, n, 1)).astype(dtype)
    X, piv, info = oracle.gesv(A, B, n, 1, "row", scale=True)
    assert (info == 0).all()
    u = float(np.finfo(dtype).eps)
    for s in range(batch):
        A64 = A[s].astype(np.float64)
        x_ref = scipy.linalg.solve(A64, B[s].astype(np.float64))
        kappa = np.linalg.cond(A64, np.inf)
        err = np.abs(X[s] - x_ref).max() / np.abs(x_ref).max()
        assert err <= 50 * n * kappa * u, (s, err)
    LU, ipiv, finfo, _ = oracle.getrf(A, n, "row", scale=True)
    gamma = n * u / (1 - n * u)
    for s in range(batch):
        L = np.tril(LU[s].astype(np.float64), -1) + np.eye(n)
        U = np.triu(LU[s].astype(np.float64))
        PA = A[s].astype(np.float64).copy()
        for k in range(n):
            PA[[k, ipiv[s, k]]] = PA[[ipiv[s, k], k]]
        bound = 2 * gamma * np.abs(np.abs(L) @ np.abs(U)).max() + 4 * u * np.abs(U).max()
        assert np.abs(PA - L @ U).max() <= bound, s
    # the zero matrix is left unscaled: a zero pivot at step 1, not 0/0
    Xz, _, iz = oracle.gesv(np.zeros((1, n, n), dtype), np.ones((1, n, 1), dtype), n, 1, "row",
                            scale=True)
    assert iz[0] == 1


@pytest.mark.parametrize("dtype", DTYPES)
def test_cholesky_nonfinite_statuses(dtype):
    rng = np.random.default_rng(45)
    n = 5
    L0, A, x, b = _exact_spd(rng, n, 1)
    A = A.astype(dtype)
    b = b.astype(dtype)
    An = A.copy()
    An[2, 3] = np.nan          # non-finite and not symmetric: -1 comes first
    Ai = A.copy()
    Ai[1, 1] = np.inf
    _, info = oracle.potrf(np.stack([A, An, Ai]), n, "row")
    assert list(info) == [0, -1, -1]
    bn = b.copy()
    bn[4, 0] = np.nan
    X, info = oracle.posv(np.stack([A, A]), np.stack([b, bn]), n, 1, "row")
    assert list(info) == [0, -1] and (X[1] == 0).all()
    # the shift overflows the first diagonal entry: s = inf > 0, L(0,0) = inf
    M = _fmax(dtype)
    Ah = np.array([[[M, 1], [1, 1]]], dtype)
    L, info = oracle.potrf(Ah, 2, "row", shift=M)
    assert info[0] == -3 and (L == 0).all()
    # finite factor, solution out of range: x = b / (L L^T) = 2^100 / 2^-1000
    e_small, e_big = (-1000, 100) if dtype == np.float64 else (-120, 20)
    X, info = oracle.posv(np.array([[[2.0 ** e_small]]], dtype),
                          np.array([[[2.0 ** e_big]]], dtype), 1, 1, "row")
    assert info[0] == -3 and X[0, 0, 0] == 0
    # a non-positive pivot comes before -3
    Aneg = np.array([[[-1, 0], [0, 1]]], dtype)
    assert oracle.potrf(Aneg, 2, "row")[1][0] == 1


# ----------------------------------------------------------------- potrs


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_potrs_exact_integer_factors(dtype, layout):
    """An integer L with a diagonal of powers of two and b = L L^T x for an
    integer x: both substitutions meet exact quotients only, so x comes out
    exactly; the entries above the diagonal are not read."""
    rng = np.random.default_rng(51)
    for n, nrhs in [(1, 1), (3, 2), (7, 1), (10, 4)]:
        L, A, x, b = _exact_spd(rng, n, nrhs)
        Lg = L.astype(dtype) + np.triu(rng.integers(5, 9, (n, n)), 1).astype(dtype)
        X = oracle.potrs(oracle.to_storage(Lg[None], layout),
                         oracle.rhs_to_storage(b[None].astype(dtype), layout), n, nrhs, layout)
        np.testing.assert_array_equal(oracle.rhs_from_storage(X, layout, n, nrhs)[0],
                                      x.astype(dtype), err_msg=f"n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_potrs_matches_lapack_and_posv(dtype):
    """Against LAPACK's potrs (scipy cho_solve on the same factor) within the
    working-precision bound; potrf then potrs is posv bit for bit (the same
    operations in the same order); a failed factorization (L all +0.0)
    gives X = +0.0."""
    rng = np.random.default_rng(52)
    n, nrhs, batch = 9, 3, 20
    G = rng.standard_normal((batch, n, n))
    A = (G @ G.transpose(0, 2, 1) / n + np.eye(n)).astype(dtype)
    A = np.tril(A) + np.tril(A, -1).transpose(0, 2, 1)
    B = rng.standard_normal((batch, n, nrhs)).astype(dtype)
    L, info = oracle.potrf(A, n, "row")
    assert (info == 0).all()
    X = oracle.potrs(L, B, n, nrhs, "row")
    Xp, _ = oracle.posv(A, B, n, nrhs, "row")
    np.testing.assert_array_equal(X, Xp)
    u = float(np.finfo(dtype).eps)
    for s in range(batch):
        ref = scipy.linalg.cho_solve((L[s].astype(np.float64), True), B[s].astype(np.float64))
        kappa = np.linalg.cond(A[s].astype(np.float64), np.inf)
        assert np.abs(X[s] - ref).max() / np.abs(ref).max() <= 20 * n * kappa * u
    Xz = oracle.potrs(np.zeros((2, n, n), dtype), B[:2], n, nrhs, "row")
    assert (Xz == 0).all() and not np.signbit(Xz).any()
