"""GPU: the float64 back substitution.  From registers (one right-hand
side, 4- and 16-lane groups) it forms each x_k from a reciprocal of U(k,k)
made before the chain and checks afterwards that this was the division
sequence's own result, solving again by division where it was not; whole-
wave groups (n = 24 and 32 when forced to them here, n = 64) divide with U
read from the packed LDS triangle.  Every route must give the oracle's
IEEE quotients bit for bit.

Inputs: well-conditioned random systems (the shortcut holds), and the same
systems with right-hand sides of 2^-1000 and exactly zero (numerators the
division sequence scales or treats specially), with A scaled by 2^1000
(large divisors) and by 2^-1000 (small ones), and single systems of each
kind placed among ordinary ones, so that one wave takes the second route
while its neighbours do not.  X, piv and info are compared with the oracle
bit for bit ("solver_static.hpp File Reference", Detailed Description: x_k
by division, in order; "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the
unchanged numerical and failure contract), except the sign of an exact
zero: the kernels give every row of a register slot the panel's rank-1
updates, and a row the elimination leaves alone takes them with multiplier
zero, an exact zero product whose addition changes no other value but
turns a -0 into +0.  Zero right-hand sides with signed entries show it, so
zeros are compared by value and everything else by its bits.
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


def _sizes(n, monkeypatch):
    out = []
    for t in (4, 16, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_gesv(tdls.F64, tdls.ROW_MAJOR, n, 1, 1)
        if rc == 0:
            out.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return out


def _systems(n, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((64, n, n)) + n * np.eye(n)
    B = rng.standard_normal((64, n, 1))
    As, Bs = [A], [B]
    for sa, sb in ((1.0, 2.0 ** -1000), (1.0, 0.0), (2.0 ** 1000, 1.0), (2.0 ** -1000, 1.0),
                   (2.0 ** 1000, 2.0 ** -1000)):
        As.append(A * sa)
        Bs.append(B * sb)
        # one such system among ordinary ones
        A1, B1 = A.copy(), B.copy()
        A1[37] *= sa
        B1[37] *= sb
        As.append(A1)
        Bs.append(B1)
    return np.concatenate(As), np.concatenate(Bs)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [5, 8, 16, 24, 32, 64])
def test_back_substitution_quotients(n, layout, monkeypatch):
    A, B = _systems(n, 300 + n)
    A_st = oracle.to_storage(A, layout)
    B_st = oracle.rhs_to_storage(B, layout)
    Xo, pivo, info_o = oracle.gesv(A_st, B_st, n, 1, layout)
    for T in _sizes(n, monkeypatch):
        what = f"n={n} {layout} T={T} batch={A.shape[0]}"
        print(f"[back substitution] {what}", flush=True)
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(T))
        X, piv, info = tdls.gesv_batched(torch.from_numpy(np.ascontiguousarray(A_st)).to(DEV),
                                         torch.from_numpy(np.ascontiguousarray(B_st)).to(DEV),
                                         layout)
        torch.cuda.synchronize()
        monkeypatch.delenv("TDLS_GROUP_SIZE")
        np.testing.assert_array_equal(info.cpu().numpy(), info_o, err_msg=what)
        np.testing.assert_array_equal(piv.cpu().numpy(), pivo, err_msg=what)
        Xg = X.cpu().numpy()
        # adding +0.0 maps -0 to +0 and leaves every other value as it is
        np.testing.assert_array_equal((Xg + 0.0).view(np.uint64),
                                      (np.ascontiguousarray(Xo) + 0.0).view(np.uint64),
                                      err_msg=what)
