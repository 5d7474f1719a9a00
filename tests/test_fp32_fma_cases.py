"""The float32 single-rounding inputs (tests/fp32_fma_cases.py) discriminate,
and the oracle rounds once: CPU only."""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import fp32_fma_cases as fc
import oracle


def test_triple_discriminates():
    exact = -Fraction(float(fc.L)) * Fraction(float(fc.U)) + Fraction(float(fc.A_))
    assert fc.bits(fc.round_f32(exact)) == fc.SINGLE
    twice = np.float32(float(exact))          # nearest float64, then float32
    assert fc.bits(twice) == fc.DOUBLE


def test_oracle_rounds_once_at_every_site():
    for n in (3, 8, 16, 32, 64):
        for name, A, b, checks in fc.gesv_cases(n):
            A_st = oracle.to_storage(A[None], "row")
            LU, piv, info, _ = oracle.getrf(A_st, n, "row")
            X, _, xinfo = oracle.gesv(A_st, b[None, :, None], n, 1, "row")
            assert info[0] == 0 and xinfo[0] == 0, name
            for chk in checks:
                if chk[0] == "neg":
                    (r1, c1), (r2, c2) = chk[1], chk[2]
                    assert fc.bits(LU[0, r2, c2]) == fc.bits(-LU[0, r1, c1]), name
                elif chk[0][0] == "x":
                    assert fc.bits(X.reshape(n)[chk[0][1]]) == chk[1], name
                else:
                    r, c = chk[0]
                    assert fc.bits(LU[0, r, c]) == chk[1], (name, n)
    # getrs and posv sites
    n = 8
    LUm = np.eye(n, dtype=np.float32)
    LUm[1, 0] = fc.L
    b = np.zeros(n, np.float32)
    b[0], b[1] = fc.U, fc.A_
    X = oracle.getrs(oracle.to_storage(LUm[None], "row"), np.arange(n, dtype=np.int32)[None],
                     b[None, :, None], n, 1, "row")
    assert fc.bits(X.reshape(n)[1]) == fc.SINGLE
    S = np.eye(n, dtype=np.float32)
    S[0, 1] = S[1, 0] = fc.L
    X, info = oracle.posv(oracle.to_storage(S[None], "row"), b[None, :, None], n, 1, "row")
    assert info[0] == 0 and fc.bits(X.reshape(n)[1]) == fc.SINGLE
