"""GPU parity where exact magnitude ties decide the pivots of non-singular
systems: the lowest current row position must win ("ruSOLVER：小矩阵 kernel
优化（实验性）", section on the unchanged numerical and failure contract:
ties to the lowest row number).

Inputs (tests/ties.py): dyadic P^T L U systems, whose eliminations tie
exactly at many steps, and ties planted at chosen steps (before, at and
after the steps where the kernels put rows back in position order), in
float64 also candidates sharing the largest high word with different low
words.  The CPU test tests/test_tie_inputs.py shows that these inputs put
tied rows on two slots of one lane, on different lanes, and with the lower
position on the higher lane, for every group size built.

Every group size built for a shape is run (TDLS_GROUP_SIZE), in both
layouts, through gesv and getrf.  Bar: info bit-exact, piv bit-exact on
every system (the gap margin does not apply: ties, not rounding, decide),
X within the normwise tolerance on kappa <= 1e3 systems and the scaled
residual <= 10; getrf's factors bit for bit the oracle's (both sides take
the same IEEE operations in the same order).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import parity
import ties
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


def _group_sizes(dtype, n, nrhs, monkeypatch):
    out = []
    for t in (4, 16, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_gesv(tdls.F64 if dtype == "f64" else tdls.F32, tdls.ROW_MAJOR, n,
                                    nrhs, 1)
        if rc == 0:
            out.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return out


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n,dtype,nrhs", ties.SHAPES)
def test_ties_decide_pivots(n, dtype, nrhs, layout, monkeypatch):
    npdt = np.float32 if dtype == "f32" else np.float64
    A = ties.tie_batch(n, dtype)
    rng = np.random.default_rng(n + nrhs)
    B = rng.uniform(-1, 1, (A.shape[0], n, nrhs)).astype(npdt)
    A_st = oracle.to_storage(A, layout)
    B_st = oracle.rhs_to_storage(B, layout)
    LUo, ipo, info_o, _ = oracle.getrf(np.ascontiguousarray(A_st), n, layout)
    assert (info_o == 0).all()
    for T in _group_sizes(dtype, n, nrhs, monkeypatch):
        what = f"{dtype} {layout} n={n} nrhs={nrhs} T={T} batch={A.shape[0]}"
        print(f"[ties] {what}", flush=True)
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
        Ad = torch.from_numpy(np.ascontiguousarray(A_st)).to(DEV)
        Bd = torch.from_numpy(np.ascontiguousarray(B_st)).to(DEV)
        X, piv, info = tdls.gesv_batched(Ad, Bd, layout)
        LU, fpiv, finfo = tdls.getrf_batched(Ad, layout)
        torch.cuda.synchronize()
        monkeypatch.delenv("TDLS_GROUP_SIZE")
        rep = parity.compare(A_st, B_st, X.cpu().numpy(), piv.cpu().numpy(), info.cpu().numpy(),
                             n, nrhs, layout, piv_all=True)
        print(f"[ties] {what}: {rep}", flush=True)
        assert rep.info_mismatch == 0, what
        assert rep.piv_checked == A.shape[0], what
        assert rep.piv_mismatch_margin == 0, what
        assert rep.x_max_err <= rep.x_tol, what
        assert rep.resid_max <= parity.RESID_TOL, what
        np.testing.assert_array_equal(finfo.cpu().numpy(), info_o, err_msg=what)
        np.testing.assert_array_equal(fpiv.cpu().numpy(), ipo, err_msg=what)
        LUg = oracle.from_storage(LU.cpu().numpy().reshape(-1, n * n), layout, n)
        np.testing.assert_array_equal(LUg, LUo, err_msg=what)
