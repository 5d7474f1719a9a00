"""GPU parity of the LU solves that run panels of two columns for one more
wave per SIMD (lu_min_waves: float64 n = 32 with one right-hand side,
n = 24 with up to four, n = 48 with four or eight, float32 n = 32 with
eight), at the kernel's own size and ragged below it, in both layouts,
against the oracle bit for bit: solution, piv and info ("solver_static.hpp
File Reference", Detailed Description: the elimination order, which the
panel width leaves unchanged).  Exact zeros are compared by value (the
sign of a zero result is not fixed: the kernels add exact zero products to
rows the elimination leaves alone).  The group size is forced, so small
batches do not move to the wider group.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import dense_linear_solvers_amd as tdls

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (dtype, kernel size N, right-hand sides to run, group size)
SHAPES = [
    ("f64", 32, (1,), 16),
    ("f64", 24, (1, 2, 3, 4), 16),
    ("f64", 48, (3, 4, 5, 8), 64),
    ("f32", 32, (5, 8), 16),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tdls.load_library()
    yield
    torch.cuda.synchronize()


def _plus_zero_bits(x):
    x = np.ascontiguousarray(x)
    return (x + x.dtype.type(0)).view(np.uint64 if x.dtype == np.float64 else np.uint32)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}-N{s[1]}-T{s[3]}")
def test_narrow_panel_shapes(shape, layout, monkeypatch):
    dtype, N, nrhs_list, T = shape
    npt = np.float64 if dtype == "f64" else np.float32
    rng = np.random.default_rng(900 + N)
    batch = 517
    for n in (N, N - 3):
        for nrhs in nrhs_list:
            A = (rng.standard_normal((batch, n, n)) + np.eye(n)).astype(npt)
            B = rng.standard_normal((batch, n, nrhs)).astype(npt)
            A[11, :, 2] = 0                        # a zero pivot: a failed system
            A_st = oracle.to_storage(A, layout)
            B_st = oracle.rhs_to_storage(B, layout)
            Xo, pivo, info_o = oracle.gesv(A_st, B_st, n, nrhs, layout)
            what = f"{dtype} {layout} n={n} nrhs={nrhs} T={T} batch={batch}"
            print(f"[narrow panels] {what}", flush=True)
            monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
            plan = tdls.plan_gesv(dtype, layout, n, nrhs, batch)
            assert plan["group_size"] == T and plan["n_kernel"] == N, (what, plan)
            X, piv, info = tdls.gesv_batched(torch.from_numpy(np.ascontiguousarray(A_st)).to(DEV),
                                             torch.from_numpy(np.ascontiguousarray(B_st)).to(DEV),
                                             layout)
            torch.cuda.synchronize()
            monkeypatch.delenv("TDLS_GROUP_SIZE")
            np.testing.assert_array_equal(info.cpu().numpy(), info_o, err_msg=what)
            assert info_o[11] == 3, what
            np.testing.assert_array_equal(piv.cpu().numpy(), pivo, err_msg=what)
            np.testing.assert_array_equal(_plus_zero_bits(X.cpu().numpy()), _plus_zero_bits(Xo),
                                          err_msg=what)
