"""GPU parity of the LU kernels on systems at the edges of the float64
range, side by side with ordinary ones: gesv's solution, piv and info and
getrf's factors must be the oracle's bit for bit ("solver_static.hpp File
Reference", Detailed Description: multipliers by division; "ruSOLVER：小矩阵
kernel 优化（实验性）", section on the unchanged numerical and failure
contract), for every kernel size, group size and both layouts.

Inputs: ordinary systems with, at the first, a middle and the last (ragged)
wave of the batch, systems whose steps reach far from 1 in magnitude: a
tiny row (candidates below 2^-500), a huge matrix (pivots above 2^500), an
exact +0 and a -0 entry in the first column, a zero column (a zero pivot),
a NaN, and a matrix scaled so that only the later steps' candidates are
tiny.  These are where a division shortcut would part from IEEE division
(the compiler's division sequence rescales operands and fixes up results
there).  Exact zeros are compared by value (the sign of a zero result is
not fixed: the kernels add exact zero products to rows the elimination
leaves alone); every other value by its bits.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import dense_linear_solvers_amd as tdls

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tdls.load_library()
    yield
    torch.cuda.synchronize()


def _sizes(n, nrhs, monkeypatch):
    out = []
    for t in (4, 16, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_gesv(tdls.F64, tdls.ROW_MAJOR, n, nrhs, 1)
        if rc == 0:
            out.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return out


def _systems(n, nrhs, batch, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((batch, n, n)) + np.eye(n)
    B = rng.standard_normal((batch, n, nrhs))
    spots = [0, batch // 2, batch - 1]
    kinds = ["tiny_row", "huge", "plus_zero", "minus_zero", "zero_col", "nan", "late_tiny"]
    for i, s in enumerate(spots * 3):
        kind = kinds[i % len(kinds)]
        s = min(s + i // len(spots), batch - 1)
        if kind == "tiny_row":
            A[s, 1] *= 2.0 ** -600
        elif kind == "huge":
            A[s] *= 2.0 ** 600
        elif kind == "plus_zero":
            A[s, 2, 0] = 0.0
        elif kind == "minus_zero":
            A[s, 2, 0] = -0.0
        elif kind == "zero_col":
            A[s, :, 1] = 0.0
        elif kind == "nan":
            A[s, 3, 2] = np.nan
        else:
            # columns from n/2 on scaled down: late steps see tiny candidates
            A[s, :, n // 2:] *= 2.0 ** -560
    return A, B


def _zero_as_plus(x):
    return (np.ascontiguousarray(x, dtype=np.float64) + 0.0).view(np.uint64)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n,nrhs", [(8, 1), (16, 1), (24, 1), (32, 1), (48, 1), (64, 1),
                                    (32, 3), (64, 8), (13, 1)])
def test_extreme_range_systems(n, nrhs, layout, monkeypatch):
    batch = 517
    A, B = _systems(n, nrhs, batch, 700 + n + nrhs)
    A_st = oracle.to_storage(A, layout)
    B_st = oracle.rhs_to_storage(B, layout)
    Xo, pivo, info_o = oracle.gesv(A_st, B_st, n, nrhs, layout)
    LUo, ipo, finfo_o, _ = oracle.getrf(A_st, n, layout)
    bad = finfo_o != 0
    for T in _sizes(n, nrhs, monkeypatch):
        what = f"n={n} nrhs={nrhs} {layout} T={T} batch={batch}"
        print(f"[extreme range] {what}", flush=True)
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
        X, piv, info = tdls.gesv_batched(torch.from_numpy(np.ascontiguousarray(A_st)).to(DEV),
                                         torch.from_numpy(np.ascontiguousarray(B_st)).to(DEV),
                                         layout)
        torch.cuda.synchronize()
        info_h = info.cpu().numpy()
        np.testing.assert_array_equal(info_h, info_o, err_msg=what)
        np.testing.assert_array_equal(piv.cpu().numpy(), pivo, err_msg=what)
        np.testing.assert_array_equal(_zero_as_plus(X.cpu().numpy()), _zero_as_plus(Xo),
                                      err_msg=what)
        if nrhs == 1:
            LU, fpiv, finfo = tdls.getrf_batched(
                torch.from_numpy(np.ascontiguousarray(A_st)).to(DEV), layout)
            torch.cuda.synchronize()
            finfo_h = finfo.cpu().numpy()
            np.testing.assert_array_equal(finfo_h, finfo_o, err_msg=what)
            LUg = oracle.from_storage(LU.cpu().numpy(), layout, n)
            # failed factorizations are +0.0 with pivots -1 (the contract)
            assert (LUg[bad] == 0).all() and (fpiv.cpu().numpy()[bad] == -1).all(), what
            np.testing.assert_array_equal(_zero_as_plus(LUg[~bad]), _zero_as_plus(LUo[~bad]),
                                          err_msg=what)
            np.testing.assert_array_equal(fpiv.cpu().numpy()[~bad], ipo[~bad], err_msg=what)
        monkeypatch.delenv("TDLS_GROUP_SIZE")
