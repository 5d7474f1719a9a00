"""GPU: float32 kernels round each fused multiply-add once.

On the inputs of tests/fp32_fma_cases.py a multiply-add computed in float64
and rounded to float32 gives other bits than the float32 fma the oracle
uses.  Every kernel size (n = 8 .. 64), every group size built for it, both
layouts, one to four right-hand sides: gesv, getrf, getrs (from the
oracle's factors) and posv must give the oracle's bits at the sites the
cases aim at, and the oracle's outputs everywhere.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fp32_fma_cases as fc
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


def _sizes(op, n, nrhs, monkeypatch):
    out = []
    for t in (4, 16, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_op(tdls._binding._OPS[op], tdls.F32, tdls.ROW_MAJOR, n, nrhs, 1)
        if rc == 0:
            out.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return out


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [8, 16, 24, 32, 48, 64])
def test_single_rounding_every_site(n, layout, monkeypatch):
    for nrhs in (1, 2, 4):
        for name, A, b, checks in fc.gesv_cases(n):
            B = np.repeat(b[:, None], nrhs, axis=1)[None]
            A_st = oracle.to_storage(A[None], layout)
            B_st = oracle.rhs_to_storage(B, layout)
            LUo, ipo, info_o, _ = oracle.getrf(A_st, n, layout)
            Xo, pivo, xinfo_o = oracle.gesv(A_st, B_st, n, nrhs, layout)
            for T in _sizes("gesv", n, nrhs, monkeypatch):
                what = f"{name} n={n} nrhs={nrhs} {layout} T={T}"
                print(f"[fp32-fma] {what}", flush=True)
                monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
                X, piv, info = tdls.gesv_batched(_dev(A_st), _dev(B_st), layout)
                LU, fpiv, finfo = (tdls.getrf_batched(_dev(A_st), layout) if nrhs == 1
                                   else (None, None, None))
                torch.cuda.synchronize()
                monkeypatch.delenv("TDLS_GROUP_SIZE")
                assert info.item() == xinfo_o[0] == 0, what
                np.testing.assert_array_equal(piv.cpu().numpy(), pivo, err_msg=what)
                Xg = oracle.rhs_from_storage(X.cpu().numpy(), layout, n, nrhs)
                Xr = oracle.rhs_from_storage(Xo, layout, n, nrhs)
                assert (Xg.view(np.uint32) == Xr.view(np.uint32)).all(), what
                if LU is not None:
                    LUg = oracle.from_storage(LU.cpu().numpy(), layout, n)
                    np.testing.assert_array_equal(fpiv.cpu().numpy(), ipo, err_msg=what)
                    assert (LUg.view(np.uint32) == LUo.view(np.uint32)).all(), what
                for chk in checks:
                    if chk[0] == "neg" or chk[0][0] == "x" or LU is None:
                        continue
                    r, c = chk[0]
                    assert fc.bits(LUg[0, r, c]) == chk[1], what


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [8, 16, 24, 32, 48, 64])
def test_single_rounding_getrs_posv(n, layout, monkeypatch):
    b = np.zeros(n, np.float32)
    b[0], b[1] = fc.U, fc.A_
    LUm = np.eye(n, dtype=np.float32)
    LUm[1, 0] = fc.L
    S = np.eye(n, dtype=np.float32)
    S[0, 1] = S[1, 0] = fc.L
    for nrhs in (1, 2, 4):
        B_st = oracle.rhs_to_storage(np.repeat(b[:, None], nrhs, axis=1)[None], layout)
        piv = np.arange(n, dtype=np.int32)[None]
        LU_st = oracle.to_storage(LUm[None], layout)
        S_st = oracle.to_storage(S[None], layout)
        Xr_o = oracle.getrs(LU_st, piv, B_st, n, nrhs, layout)
        Xp_o, pinfo_o = oracle.posv(S_st, B_st, n, nrhs, layout)
        assert pinfo_o[0] == 0
        for op in ("getrs", "posv"):
            for T in _sizes(op, n, nrhs, monkeypatch):
                what = f"{op} n={n} nrhs={nrhs} {layout} T={T}"
                print(f"[fp32-fma] {what}", flush=True)
                monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
                if op == "getrs":
                    X = tdls.getrs_batched(_dev(LU_st), _dev(piv), _dev(B_st), layout)
                    ref = Xr_o
                else:
                    X, info = tdls.posv_batched(_dev(S_st), _dev(B_st), layout)
                    ref = Xp_o
                torch.cuda.synchronize()
                monkeypatch.delenv("TDLS_GROUP_SIZE")
                Xg = oracle.rhs_from_storage(X.cpu().numpy(), layout, n, nrhs)
                Xr = oracle.rhs_from_storage(ref, layout, n, nrhs)
                assert (Xg.view(np.uint32) == Xr.view(np.uint32)).all(), what
                assert fc.bits(Xg[0, 1, 0]) == fc.SINGLE, what
