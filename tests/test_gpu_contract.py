"""GPU parity of the ruSOLVER contract extensions through the C interface:
the non-finite statuses (-1 for a non-finite input entry, -3 for a
non-finite computed value, after the positive status of a failed pivot) of
gesv, getrf, potrf and posv, and the whole-matrix max-abs scaling of gesv
and getrf (tdls_*_batched_ex), against the CPU oracle.

Bar: info bit-exact on every system; a failed system has X (or LU, L) all
+0.0 and piv all -1; the other systems meet the bar of the plain parity
tests (piv on gap-margin systems, X within the normwise tolerance where
kappa <= 1e3, scaled residual <= 10).  Inputs: seeded random batches with
NaN and infinities planted in chosen entries, matrices scaled near the top
of the floating-point range so that the elimination overflows in some
systems and not in others, and the hand-built cases of the oracle's pins
embedded in identity blocks.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import parity
import dense_linear_solvers_amd as tdls
from dense_linear_solvers_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(dt):
    return np.float32 if dt == "f32" else np.float64


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tdls.load_library()
    yield
    torch.cuda.synchronize()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_gesv(A_st, B_st, layout, scale=False):
    X, piv, info = tdls.gesv_batched(_dev(A_st), _dev(B_st), layout, scale=scale)
    torch.cuda.synchronize()
    return X.cpu().numpy(), piv.cpu().numpy(), info.cpu().numpy()


def gpu_getrf(A_st, layout, scale=False):
    LU, piv, info = tdls.getrf_batched(_dev(A_st), layout, scale=scale)
    torch.cuda.synchronize()
    return LU.cpu().numpy(), piv.cpu().numpy(), info.cpu().numpy()


def gpu_potrf(A_st, layout, shift=0.0):
    L, info = tdls.potrf_batched(_dev(A_st), layout, shift)
    torch.cuda.synchronize()
    return L.cpu().numpy(), info.cpu().numpy()


def gpu_posv(A_st, B_st, layout, shift=0.0):
    X, info = tdls.posv_batched(_dev(A_st), _dev(B_st), layout, shift)
    torch.cuda.synchronize()
    return X.cpu().numpy(), info.cpu().numpy()


def check_gesv(A_st, B_st, n, nrhs, layout, what, scale=False):
    X, piv, info = gpu_gesv(A_st, B_st, layout, scale)
    rep = parity.compare(A_st, B_st, X, piv, info, n, nrhs, layout, scale=scale)
    print(f"{what}: {rep} statuses={np.unique(info, return_counts=True)}", flush=True)
    assert rep.info_mismatch == 0, what
    assert rep.piv_mismatch_margin == 0, what
    assert rep.failed_bad_outputs == 0, what
    assert rep.x_max_err <= rep.x_tol, what
    assert rep.resid_max <= parity.RESID_TOL, what
    return X, piv, info


def check_getrf(A_st, n, layout, what, scale=False):
    LU, piv, info = gpu_getrf(A_st, layout, scale)
    LUo, ipo, info_o, gap = oracle.getrf(A_st, n, layout, scale=scale)
    assert (info == info_o).all(), f"{what}: info {info[info != info_o]} vs {info_o[info != info_o]}"
    LUg = oracle.from_storage(LU, layout, n)
    bad = info_o != 0
    assert (LUg[bad] == 0).all() and not np.signbit(LUg[bad]).any(), what
    assert (piv[bad] == -1).all(), what
    dt = np.dtype(A_st.dtype)
    margin = ~bad & (gap >= parity.GAP_TOL[dt])
    assert (piv[margin] == ipo[margin]).all(), what
    if margin.any():
        num = np.abs(LUg[margin].astype(np.float64) - LUo[margin]).max(axis=(1, 2))
        den = np.abs(LUo[margin].astype(np.float64)).max(axis=(1, 2))
        assert (num / den).max() <= parity.X_TOL[dt], what
    return LU, piv, info


def plant_nonfinite(rng, A, B, systems):
    """NaN, +inf or -inf in one entry of A (early or late column) or of B of
    each listed system; returns the arrays (logical order)."""
    A, B = A.copy(), B.copy()
    n = A.shape[1]
    vals = [np.nan, np.inf, -np.inf]
    for i, s in enumerate(systems):
        v = vals[i % 3]
        kind = i % 4
        if kind == 0:
            A[s, rng.integers(n), rng.integers(min(4, n))] = v        # first panel
        elif kind == 1:
            A[s, rng.integers(n), n - 1 - rng.integers(max(1, n // 2))] = v
        elif kind == 2:
            A[s, rng.integers(n), rng.integers(n)] = v
        else:
            B[s, rng.integers(n), rng.integers(B.shape[2])] = v
    return A, B


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n,nrhs", [(8, 1), (13, 2), (32, 1), (24, 3), (64, 8)])
def test_nonfinite_inputs(dtype, layout, n, nrhs):
    rng = np.random.default_rng(100 + n + nrhs)
    batch = 203
    A = rng.uniform(-1, 1, (batch, n, n)).astype(_np(dtype))
    B = rng.uniform(-1, 1, (batch, n, nrhs)).astype(_np(dtype))
    systems = rng.choice(batch, size=40, replace=False)
    A, B = plant_nonfinite(rng, A, B, systems)
    # -1 outranks a zero pivot of the first panel and of a later one
    A[systems[0], :, 0] = 0
    A[systems[0], 3, n - 1] = np.nan
    A[systems[1], :, min(6, n - 1)] = 0
    A[systems[1], 0, 1] = np.inf
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X, piv, info = check_gesv(A_st, B_st, n, nrhs, layout, f"gesv {dtype} {layout} n={n}")
    assert (info[systems] == -1).sum() >= 30
    LU, lpiv, linfo = check_getrf(A_st, n, layout, f"getrf {dtype} {layout} n={n}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [8, 32, 64])
def test_overflow_statuses(dtype, layout, n):
    """Matrices near the top of the range: the elimination overflows in some
    systems (-3) and not in others; the statuses must agree exactly."""
    rng = np.random.default_rng(200 + n)
    batch = 150
    top = 1021 if dtype == "f64" else 125
    A = (rng.standard_normal((batch, n, n)) * 2.0 ** top).astype(_np(dtype))
    B = rng.standard_normal((batch, n, 1)).astype(_np(dtype))
    assert np.isfinite(A).all()
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X, piv, info = check_gesv(A_st, B_st, n, 1, layout, f"gesv overflow {dtype} {layout} n={n}")
    check_getrf(A_st, n, layout, f"getrf overflow {dtype} {layout} n={n}")


def _embed(E, n, dtype):
    k = E.shape[0]
    A = np.eye(n)
    A[:k, :k] = E
    return A.astype(dtype)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [4, 8, 32, 64])
def test_hand_built_statuses(dtype, layout, n):
    """The oracle's hand-built cases: an overflow into U (-3), a solution out
    of range (-3), a NaN candidate that must outrank an exact zero (-3, not
    a zero-pivot status), and a zero pivot after an overflow (3)."""
    npd = _np(dtype)
    M = 0.75 * float(np.finfo(npd).max)
    es, eb = (-1000, 100) if dtype == "f64" else (-120, 20)
    cases = []
    if n >= 2:
        cases.append((np.array([[1, M], [1, -M]]), -3))
        cases.append((np.array([[2.0 ** es]]), -3))
    if n >= 3:
        cases.append((np.array([[1, M, 0], [1, -M, 0], [0, 0, 0]]), 3))
    if n >= 4:
        cases.append((np.array([[1, M, 0, 0], [1, -M, 1, 0], [0, 1, 0, 1], [1, -M, 0, 0]]), -3))
    A = np.stack([_embed(E, n, npd) for E, _ in cases])
    B = np.ones((len(cases), n, 1), npd)
    B[1, 0, 0] = 2.0 ** eb
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X, piv, info = check_gesv(A_st, B_st, n, 1, layout, f"hand-built {dtype} {layout} n={n}")
    assert list(info) == [c for _, c in cases]


RECIPE_NAMES = sorted(workloads.RECIPES)


@pytest.mark.parametrize("name", RECIPE_NAMES)
def test_scaled_recipes(name):
    """Max-abs scaling on every recipe (a batch spanning many blocks with a
    ragged tail): gesv and getrf vs the oracle's scaled versions."""
    r = workloads.RECIPES[name]
    spb = tdls.plan_gesv(r.dtype, r.layout, r.n, r.nrhs, 1)["systems_per_block"]
    batch = 23 * spb + 3
    w = workloads.make(name, seed=0, batch=batch)
    check_gesv(w.A, w.B, w.n, w.nrhs, w.layout, f"scaled {name}", scale=True)
    check_getrf(w.A, w.n, w.layout, f"scaled getrf {name}", scale=True)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n,nrhs", [(8, 1), (24, 2), (32, 1), (64, 8)])
def test_scaling_by_power_of_two_is_exact(dtype, layout, n, nrhs):
    """A largest magnitude that is a power of two makes the scaling exact,
    so the scaled results are the unscaled ones, bit for bit."""
    rng = np.random.default_rng(300 + n)
    batch = 97
    A = rng.uniform(-1, 1, (batch, n, n))
    for s in range(batch):
        A[s, rng.integers(n), rng.integers(n)] = rng.choice([-1.0, 1.0])
        A[s] *= 2.0 ** int(rng.integers(-8, 9))
    A = A.astype(_np(dtype))
    B = rng.uniform(-1, 1, (batch, n, nrhs)).astype(_np(dtype))
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X0, p0, i0 = gpu_gesv(A_st, B_st, layout)
    X1, p1, i1 = gpu_gesv(A_st, B_st, layout, scale=True)
    np.testing.assert_array_equal(X1, X0)
    np.testing.assert_array_equal(p1, p0)
    np.testing.assert_array_equal(i1, i0)
    L0, q0, f0 = gpu_getrf(A_st, layout)
    L1, q1, f1 = gpu_getrf(A_st, layout, scale=True)
    np.testing.assert_array_equal(L1, L0)
    np.testing.assert_array_equal(q1, q0)


def test_scaled_edge_cases():
    """Zero matrices (not scaled: a zero pivot at step 1), a non-finite input
    under scaling (-1), and the empty batch."""
    n = 16
    A = np.zeros((3, n, n))
    A[1] = np.eye(n) * 3.0
    A[2] = np.eye(n)
    A[2, 4, 9] = np.nan
    A = A.astype(np.float64)
    B = np.ones((3, n, 2))
    X, piv, info = check_gesv(A, B, n, 2, "row", "scaled edges", scale=True)
    assert list(info) == [1, 0, -1]
    X, piv, info = tdls.gesv_batched(torch.zeros((0, n, n), dtype=torch.float64, device=DEV),
                                     torch.zeros((0, n, 1), dtype=torch.float64, device=DEV),
                                     "row", scale=True)
    assert X.shape[0] == 0


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("name", sorted(workloads.SPD_RECIPES))
def test_cholesky_nonfinite(dtype, layout, name):
    """potrf / posv: planted non-finite entries (-1, before -2), a shift
    that overflows the first diagonal entry (-3), a solution out of range
    (-3), statuses vs the oracle's exactly."""
    r = workloads.SPD_RECIPES[name]
    w = workloads.make(name, seed=0, batch=120)
    n, nrhs = w.n, w.nrhs
    A = oracle.from_storage(w.A, w.layout, n).astype(_np(dtype))
    B = oracle.rhs_from_storage(w.B, w.layout, n, nrhs).astype(_np(dtype))
    rng = np.random.default_rng(400 + n)
    systems = rng.choice(len(A), size=24, replace=False)
    A, B = plant_nonfinite(rng, A, B, systems)
    # -3: a solution out of range (a tiny leading diagonal, its right-hand
    # side large)
    es, eb = (-1000, 100) if dtype == "f64" else (-120, 20)
    t = [s for s in range(len(A)) if s not in set(systems)][:2]
    A[t[0]] = np.eye(n, dtype=A.dtype)
    A[t[0], 0, 0] = 2.0 ** es
    B[t[0]] = 1
    B[t[0], 0, :] = 2.0 ** eb
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    for shift in (0.0, 0.5):
        X, info = gpu_posv(A_st, B_st, layout, shift)
        Xo, info_o = oracle.posv(A_st, B_st, n, nrhs, layout, shift=shift)
        assert (info == info_o).all(), (name, shift, info[info != info_o], info_o[info != info_o])
        bad = info_o != 0
        Xb = X.reshape(len(A), -1)[bad]
        assert (Xb == 0).all() and not np.signbit(Xb).any()
        good = ~bad
        err = np.abs(X.reshape(len(A), -1)[good] - Xo.reshape(len(A), -1)[good]).max(axis=1)
        den = np.abs(Xo.reshape(len(A), -1)[good]).max(axis=1)
        kappa = np.linalg.cond(A[good].astype(np.float64), np.inf)
        well = kappa <= parity.KAPPA_MAX
        assert (err[well] / den[well]).max() <= parity.X_TOL[np.dtype(_np(dtype))]
        L, linfo = gpu_potrf(A_st, layout, shift)
        Lo, linfo_o = oracle.potrf(A_st, n, layout, shift=shift)
        assert (linfo == linfo_o).all(), (name, shift)
        assert (oracle.from_storage(L, layout, n)[linfo_o != 0] == 0).all()
        assert (info[systems] == -1).all()
        if shift == 0.0:        # with the shift, the tiny diagonal is gone
            assert info[t[0]] == -3
    # a shift that overflows the first diagonal entry of every system: -3
    # for the finite ones (inf on the diagonal of L), -1 for the planted
    big = float(np.finfo(_np(dtype)).max)
    A2 = A.copy()
    A2[:, 0, 0] = big
    A2_st = oracle.to_storage(A2, layout)
    L, linfo = gpu_potrf(A2_st, layout, big)
    Lo, linfo_o = oracle.potrf(A2_st, n, layout, shift=big)
    assert (linfo == linfo_o).all()
    assert (linfo_o[[s for s in range(len(A)) if s not in set(systems)]] == -3).all()
