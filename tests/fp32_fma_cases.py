"""Float32 inputs on which a single-rounded fused multiply-add and the same
operation done in float64 and rounded to float32 disagree.

The triple (l, u, a) below has fmaf(-l, u, a) = 0x3f199999 while the
float64 fma of the same operands, rounded to float32, is 0x3f19999a: the
exact value lies 2^-48 below a float32 rounding midpoint, the float64
result lands on that midpoint and the second rounding goes to even.  The
systems place this operation at each site where a kernel fuses a multiply
and an add, so a kernel that rounds twice gives different bits there than
the oracle (explicit fmaf).

  panel    A = [[1, 0, u], [l, 1, a], ...]: step 0 updates column 2, inside
           the first panel of four columns, of row 1: LU[1][2].
  pivotrow A = [[1, 0, 0, 0, 0, u], [l, 1, 0, 0, 0, a], [0, 1, 1, 0, 0, 0], ...]:
           row 1 is the pivot of step 1 (a tie with row 2, lowest position
           wins) and its column 5, outside the panel, takes step 0's update
           before it serves step 1: LU[2][5] = -LU[1][5].
  backsub  A = [[1, l], [0, 1]], b = [a, u]: x0 = fmaf(-l, u, a).
  getrs    LU = [[1, 0], [l, 1]], piv = [0, 1], b = [u, a]: y1 = fmaf(-l, u, a).
  posv     A = [[1, l], [l, 1]], b = [u, a]: L(1,1) = 1 in float32, so
           x1 = fmaf(-l, u, a).
Each is embedded in an identity of order n (rows and columns beyond the
2 or 6 used) so that every kernel size runs it.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def f32(bits: int) -> np.float32:
    return np.frombuffer(np.uint32(bits).tobytes(), np.float32)[0]


L = f32(0xB27FFFFE)      # -0x1.fffffcp-27
U = f32(0x40000001)      # 0x1.000002p+1
A_ = f32(0x3F199999)     # 0x1.333332p-1
SINGLE = 0x3F199999      # fmaf(-L, U, A_)
DOUBLE = 0x3F19999A      # the float64 fma rounded to float32


def round_f32(x: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (ties to even)."""
    f = np.float32(float(x))
    if Fraction(float(f)) == x:
        return f
    lo, hi = (np.nextafter(f, np.float32(-np.inf)), f) if Fraction(float(f)) > x else \
        (f, np.nextafter(f, np.float32(np.inf)))
    dl, dh = x - Fraction(float(lo)), Fraction(float(hi)) - x
    if dl != dh:
        return lo if dl < dh else hi
    return lo if int(np.frombuffer(lo.tobytes(), np.uint32)[0]) % 2 == 0 else hi


def bits(x) -> int:
    return int(np.frombuffer(np.float32(x).tobytes(), np.uint32)[0])


def embed(M: np.ndarray, n: int) -> np.ndarray:
    out = np.eye(n, dtype=np.float32)
    k = M.shape[0]
    out[:k, :k] = M
    return out


def gesv_cases(n: int):
    """(name, logical A [n, n], logical b [n], checks): checks are
    (row, col) of LU or ('x', i) of the solution with the expected bits, or
    ('neg', (r1, c1), (r2, c2)): LU[r2][c2] = -LU[r1][c1]."""
    out = []
    M = np.zeros((3, 3), np.float32)
    M[0, 0], M[0, 2], M[1, 0], M[1, 1], M[1, 2], M[2, 2] = 1, U, L, 1, A_, 1
    out.append(("panel", embed(M, n), np.zeros(n, np.float32), [((1, 2), SINGLE)]))
    if n >= 6:
        M = np.zeros((6, 6), np.float32)
        M[0, 0], M[0, 5] = 1, U
        M[1, 0], M[1, 1], M[1, 5] = L, 1, A_
        M[2, 1], M[2, 2] = 1, 1
        M[3, 3], M[4, 4], M[5, 5] = 1, 1, 1
        out.append(("pivotrow", embed(M, n), np.zeros(n, np.float32),
                    [((1, 5), SINGLE), ("neg", (1, 5), (2, 5))]))
    M = np.array([[1, L], [0, 1]], np.float32)
    b = np.zeros(n, np.float32)
    b[0], b[1] = A_, U
    out.append(("backsub", embed(M, n), b, [(("x", 0), SINGLE)]))
    return out
