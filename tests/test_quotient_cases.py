"""CPU pins of the hard float32 quotients in tests/f32_quotient_cases.py,
which the GPU test tests/test_gpu_f32_quotients.py puts into the kernels'
multipliers: numpy's float32 division (the reference there, through the
oracle's C division) is the exact quotient rounded to nearest even; the
hardest pairs sit at the minimal distance 1 / (D 2^25) from a midpoint; the
subnormal cases are exact midpoints or below the normal range; and the
cases are hard enough that a float64 quotient 16 ulps off rounds some of
them wrongly (a planted mistake, on the CPU).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import f32_quotient_cases as qc
from fp32_fma_cases import round_f32


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _cases():
    rng = np.random.default_rng(2024)
    return {
        "hardest_normal": qc.hardest_normal(rng, 2000),
        "hardest_normal_far": qc.hardest_normal(rng, 1000, 20, 100, d_exp=-20),
        "subnormal_midpoints": qc.subnormal_midpoints(rng, 1000),
        "underflow": qc.underflow(rng, 1000),
        "random_bits": qc.random_bits(rng, 1000),
        "edges": (np.array([0.0, -0.0, 1.0, -1.0, 3.0, 1e-45, -1e-45, 3.4e38, 1e-38, 0.0],
                           np.float32),
                  np.array([3.0, 7.0, 3.0, -3.0, 1e-45, 3.0, 1.5, 0.5, 3.4e38, -2.0],
                           np.float32)),
    }


def test_reference_division_is_correctly_rounded():
    """numpy float32 division against the exact quotient rounded to
    nearest even, on a sample of every kind of case."""
    for name, (a, d) in _cases().items():
        n = min(len(a), 300)
        with np.errstate(over="ignore"):
            q = (a[:n] / d[:n]).astype(np.float32)
        for ai, di, qi in zip(a[:n], d[:n], q):
            if not np.isfinite(qi):
                continue              # overflow: beyond the exact rounding helper
            exact = Fraction(float(ai)) / Fraction(float(di))
            want = round_f32(exact)
            if want == 0:   # the sign of a zero quotient: exclusive or of the signs
                want = np.float32(-0.0) if np.signbit(ai) != np.signbit(di) else np.float32(0.0)
            assert _bits(want) == _bits(qi), (name, ai, di)


def test_hardest_pairs_sit_at_the_minimal_distance():
    rng = np.random.default_rng(3)
    a, d = qc.hardest_normal(rng, 200)
    for ai, di in zip(a, d):
        t = abs(Fraction(float(ai)) / Fraction(float(di)))
        while t < Fraction(1, 2):
            t *= 2
        D = abs(Fraction(float(di))) / Fraction(2) ** (int(np.frexp(abs(float(di)))[1]) - 24)
        assert D.denominator == 1
        # distance from the nearest midpoint (2i+1) 2^-25 of [1/2, 1)
        scaled = t * 2 ** 25
        M = int(scaled) if int(scaled) % 2 == 1 else int(scaled) + 1
        dist = min(abs(scaled - M), abs(scaled - (M - 2)))
        assert dist == Fraction(1, int(D)), (ai, di)


def test_subnormal_cases():
    rng = np.random.default_rng(5)
    a, d = qc.subnormal_midpoints(rng, 300)
    for ai, di in zip(a, d):
        q = Fraction(float(ai)) / Fraction(float(di))
        scaled = q * 2 ** 150
        assert scaled.denominator == 1 and scaled.numerator % 2 == 1     # M 2^-150, M odd
    a, d = qc.underflow(rng, 300)
    assert (np.abs(a.astype(np.float64) / d.astype(np.float64)) < 2.0 ** -126).all()
    assert (np.abs(a) <= np.abs(d)).all()


def test_cases_show_a_quotient_that_is_not_correctly_rounded():
    """Planted mistake: the float64 quotient moved 16 float64 ulps and
    rounded to float32 differs from the IEEE quotient on some hardest pairs,
    and the unmoved one rounded twice differs on some subnormal midpoints."""
    rng = np.random.default_rng(11)
    a, d = qc.hardest_normal(rng, 4000)
    ref = _bits(a / d)
    q64 = a.astype(np.float64) / d.astype(np.float64)
    for step in (np.inf, -np.inf):
        moved = q64.copy()
        for _ in range(16):
            moved = np.nextafter(moved, step)
        assert (_bits(moved.astype(np.float32)) != ref).any()
    a, d = qc.subnormal_midpoints(rng, 2000)
    ref = _bits(a / d)
    y = 1.0 / d.astype(np.float64)                       # inexact for d = 2 D, D > 1
    assert (_bits((a.astype(np.float64) * y).astype(np.float32)) != ref).any()


def test_matrices_form_the_quotients():
    """The kernels' inputs: column k0 below the diagonal holds the numerators,
    the divisor is the largest of the column (LU) or the float32 square root
    of the diagonal (Cholesky), everything else is the identity (or a
    dominant diagonal)."""
    rng = np.random.default_rng(9)
    for kind in ("hardest", "submid", "underflow", "random"):
        for n, k0 in ((8, 0), (24, 5), (64, 33)):
            A = qc.lu_column_matrix(rng, n, k0, kind)
            col = A[k0:, k0]
            assert np.abs(col[1:]).max() < abs(col[0])
            B = A.copy()
            B[k0 + 1:, k0] = 0
            assert (B == np.diag(np.diag(B))).all()
            S = qc.chol_column_matrix(rng, n, k0, kind)
            assert (S == S.T).all()
            assert np.sqrt(S[k0, k0]) ** 2 == S[k0, k0] or kind != "hardest"
            assert np.linalg.eigvalsh(S.astype(np.float64)).min() > 0
