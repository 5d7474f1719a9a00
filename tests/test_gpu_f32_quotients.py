"""GPU: float32 multipliers and Cholesky quotients are the IEEE quotients,
bit for bit, on the float32 quotients hardest to round ("ruSOLVER：小矩阵
kernel 优化（实验性）", section on the unchanged numerical and failure
contract: exact quotients, no reciprocal approximation).

Inputs (tests/f32_quotient_cases.py, pinned on the CPU in
tests/test_quotient_cases.py): matrices whose step k0 divides a column of
numerators by one divisor, with quotients at the minimal distance from a
float32 rounding midpoint, exact subnormal midpoints among ordinary
quotients, quotients that underflow, and ordinary ones; k0 before, at and
after the steps where the kernels put rows back in position order, so that
one to all of a lane's slots hold such rows.  Every size, every group size
built for it, both layouts: getrf's factors and potrf's L bit for bit the
oracle's, and gesv's and posv's solutions too (the same IEEE operations in
the same order).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import f32_quotient_cases as qc
import oracle
import dense_linear_solvers_amd as tdls

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KINDS = ("hardest", "submid", "underflow", "random")


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tdls.load_library()
    yield
    torch.cuda.synchronize()


def _sizes(op, n, nrhs, monkeypatch):
    out = []
    for t in (4, 16, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_op(tdls._binding._OPS[op], tdls.F32, tdls.ROW_MAJOR, n, nrhs, 1)
        if rc == 0:
            out.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return out


def _steps(n):
    return sorted(k for k in {0, 1, 3, 4, 5, 8, 15, 16, 17, 31, 32, 33, n - 3, n - 2}
                  if 0 <= k <= n - 2)


def _batch(make, n, seed):
    rng = np.random.default_rng(seed)
    mats = [make(rng, n, k0, kind) for k0 in _steps(n) for kind in KINDS for _ in range(5)]
    return np.stack(mats)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [8, 16, 24, 32, 48, 64])
def test_lu_multipliers_are_ieee_quotients(n, layout, monkeypatch):
    A = _batch(qc.lu_column_matrix, n, 100 + n)
    nrhs = 2
    B = np.random.default_rng(n).uniform(-1, 1, (A.shape[0], n, nrhs)).astype(np.float32)
    A_st = oracle.to_storage(A, layout)
    B_st = oracle.rhs_to_storage(B, layout)
    LUo, ipo, info_o, _ = oracle.getrf(A_st, n, layout)
    Xo, pivo, xinfo_o = oracle.gesv(A_st, B_st, n, nrhs, layout)
    assert (info_o == 0).all()
    sizes = sorted(set(_sizes("getrf", n, 1, monkeypatch)) | set(_sizes("gesv", n, nrhs, monkeypatch)))
    for T in sizes:
        what = f"n={n} {layout} T={T} batch={A.shape[0]}"
        print(f"[quotients] LU {what}", flush=True)
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
        if T in _sizes("getrf", n, 1, monkeypatch):
            monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
            LU, piv, info = tdls.getrf_batched(_dev(A_st), layout)
            LUg = oracle.from_storage(LU.cpu().numpy().reshape(-1, n * n), layout, n)
            np.testing.assert_array_equal(info.cpu().numpy(), info_o, err_msg=what)
            np.testing.assert_array_equal(piv.cpu().numpy(), ipo, err_msg=what)
            np.testing.assert_array_equal(LUg.view(np.uint32), LUo.view(np.uint32), err_msg=what)
        if T in _sizes("gesv", n, nrhs, monkeypatch):
            monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
            X, piv, info = tdls.gesv_batched(_dev(A_st), _dev(B_st), layout)
            np.testing.assert_array_equal(info.cpu().numpy(), xinfo_o, err_msg=what)
            np.testing.assert_array_equal(piv.cpu().numpy(), pivo, err_msg=what)
            np.testing.assert_array_equal(X.cpu().numpy().view(np.uint32),
                                          np.ascontiguousarray(Xo).view(np.uint32), err_msg=what)
        monkeypatch.delenv("TDLS_GROUP_SIZE", raising=False)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [8, 16, 24, 32, 48, 64])
def test_cholesky_quotients_are_ieee(n, layout, monkeypatch):
    A = _batch(qc.chol_column_matrix, n, 200 + n)
    nrhs = 2
    B = np.random.default_rng(n + 1).uniform(-1, 1, (A.shape[0], n, nrhs)).astype(np.float32)
    A_st = oracle.to_storage(A, layout)
    B_st = oracle.rhs_to_storage(B, layout)
    Lo, info_o = oracle.potrf(A_st, n, layout)
    Xo, xinfo_o = oracle.posv(A_st, B_st, n, nrhs, layout)
    assert (info_o == 0).all()
    sizes = sorted(set(_sizes("potrf", n, 1, monkeypatch)) & set(_sizes("posv", n, nrhs, monkeypatch)))
    for T in sizes:
        what = f"n={n} {layout} T={T} batch={A.shape[0]}"
        print(f"[quotients] Cholesky {what}", flush=True)
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
        L, info = tdls.potrf_batched(_dev(A_st), layout)
        X, xinfo = tdls.posv_batched(_dev(A_st), _dev(B_st), layout)
        monkeypatch.delenv("TDLS_GROUP_SIZE")
        Lg = oracle.from_storage(L.cpu().numpy().reshape(-1, n * n), layout, n)
        np.testing.assert_array_equal(info.cpu().numpy(), info_o, err_msg=what)
        np.testing.assert_array_equal(np.tril(Lg).view(np.uint32), np.tril(Lo).view(np.uint32),
                                      err_msg=what)
        np.testing.assert_array_equal(xinfo.cpu().numpy(), xinfo_o, err_msg=what)
        np.testing.assert_array_equal(X.cpu().numpy().view(np.uint32),
                                      np.ascontiguousarray(Xo).view(np.uint32), err_msg=what)
