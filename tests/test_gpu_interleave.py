"""GPU parity of interleaved batches (the *_ex calls with interleave W):
arrays of structures of arrays (1 < W < batch, the last block ragged) and
structures of arrays (W = batch) for gesv, getrf, getrs, potrf, potrs and
posv.

Bar: the outputs are bitwise those of the plain calls on the same systems
(the arithmetic does not depend on where a system is stored; the plain
calls are checked against the oracle by the other parity tests, and one
case per operation here is also checked against the oracle directly), and
the slots of the last block past the batch are left untouched.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import layouts
import oracle
import parity
import dense_linear_solvers_amd as tdls
from dense_linear_solvers_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = -7.25


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tdls.load_library()
    yield
    torch.cuda.synchronize()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t):
    return t.cpu().numpy()


def _inputs(rng, batch, n, nrhs, dtype, spd=False):
    if spd:
        G = rng.standard_normal((batch, n, n))
        A = G @ G.transpose(0, 2, 1) / n + np.eye(n)
        A = A.astype(dtype)
        A = np.tril(A) + np.tril(A, -1).transpose(0, 2, 1)
    else:
        A = rng.uniform(-1, 1, (batch, n, n)).astype(dtype)
    B = rng.uniform(-1, 1, (batch, n, nrhs)).astype(dtype)
    return A, B


CASES = [  # (dtype, layout, n, nrhs)
    (np.float64, "col", 32, 1),
    (np.float64, "row", 64, 8),
    (np.float32, "row", 16, 4),
    (np.float32, "col", 24, 2),
    (np.float64, "row", 13, 3),
]


def _ws(batch):
    return [2, 4, 7, 64, batch]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{np.dtype(c[0]).name}-{c[1]}-n{c[2]}-r{c[3]}")
def test_interleaved_lu(case):
    dtype, layout, n, nrhs = case
    rng = np.random.default_rng(n * 10 + nrhs)
    batch = 203
    A, B = _inputs(rng, batch, n, nrhs, dtype)
    A[5, :, 2] = 0                      # a failed system keeps its record
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X0, p0, i0 = (_host(t) for t in tdls.gesv_batched(_dev(A_st), _dev(B_st), layout))
    L0, q0, f0 = (_host(t) for t in tdls.getrf_batched(_dev(A_st), layout))
    Xs0 = _host(tdls.getrs_batched(_dev(L0), _dev(q0), _dev(B_st), layout))
    assert i0[5] == 3 and f0[5] == 3
    for W in _ws(batch):
        Ai = _dev(layouts.to_interleaved(A_st, W, SENTINEL))
        Bi = _dev(layouts.to_interleaved(B_st, W, SENTINEL))
        blocks = Ai.shape[0]
        X = torch.full_like(Bi, SENTINEL)
        piv = torch.full((blocks, n, W), -77, dtype=torch.int32, device=DEV)
        info = torch.empty((batch,), dtype=torch.int32, device=DEV)
        tdls.gesv_batched(Ai, Bi, layout, out=(X, piv, info), interleave=W, batch=batch)
        Xh, ph = _host(X), _host(piv)
        np.testing.assert_array_equal(layouts.from_interleaved(Xh, batch), X0, err_msg=f"W={W}")
        np.testing.assert_array_equal(layouts.from_interleaved(ph, batch), p0)
        np.testing.assert_array_equal(_host(info), i0)
        assert (layouts.padding_of(Xh, batch) == SENTINEL).all()
        assert (layouts.padding_of(ph, batch) == -77).all()
        LU = torch.full_like(Ai, SENTINEL)
        fp = torch.full((blocks, n, W), -77, dtype=torch.int32, device=DEV)
        finfo = torch.empty((batch,), dtype=torch.int32, device=DEV)
        tdls.getrf_batched(Ai, layout, out=(LU, fp, finfo), interleave=W, batch=batch)
        LUh = _host(LU)
        np.testing.assert_array_equal(layouts.from_interleaved(LUh, batch), L0)
        np.testing.assert_array_equal(layouts.from_interleaved(_host(fp), batch), q0)
        np.testing.assert_array_equal(_host(finfo), f0)
        assert (layouts.padding_of(LUh, batch) == SENTINEL).all()
        Xs = torch.full_like(Bi, SENTINEL)
        tdls.getrs_batched(LU, fp, Bi, layout, out=Xs, interleave=W, batch=batch)
        Xsh = _host(Xs)
        np.testing.assert_array_equal(layouts.from_interleaved(Xsh, batch), Xs0)
        assert (layouts.padding_of(Xsh, batch) == SENTINEL).all()
    # the plain results against the oracle (one case per operation here)
    rep = parity.compare(A_st, B_st, X0, p0, i0, n, nrhs, layout)
    assert rep.info_mismatch == 0 and rep.failed_bad_outputs == 0
    assert rep.x_max_err <= rep.x_tol and rep.resid_max <= parity.RESID_TOL


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{np.dtype(c[0]).name}-{c[1]}-n{c[2]}-r{c[3]}")
def test_interleaved_cholesky(case):
    dtype, layout, n, nrhs = case
    rng = np.random.default_rng(n * 10 + nrhs + 1)
    batch = 150
    A, B = _inputs(rng, batch, n, nrhs, dtype, spd=True)
    A[7, 1, 2] += 1                     # not symmetric: -2
    A_st, B_st = oracle.to_storage(A, layout), oracle.rhs_to_storage(B, layout)
    X0, i0 = (_host(t) for t in tdls.posv_batched(_dev(A_st), _dev(B_st), layout, 0.25))
    L0, f0 = (_host(t) for t in tdls.potrf_batched(_dev(A_st), layout, 0.25))
    assert i0[7] == -2 and f0[7] == -2
    for W in _ws(batch):
        Ai = _dev(layouts.to_interleaved(A_st, W, SENTINEL))
        Bi = _dev(layouts.to_interleaved(B_st, W, SENTINEL))
        X = torch.full_like(Bi, SENTINEL)
        info = torch.empty((batch,), dtype=torch.int32, device=DEV)
        tdls.posv_batched(Ai, Bi, layout, 0.25, out=(X, info), interleave=W, batch=batch)
        Xh = _host(X)
        np.testing.assert_array_equal(layouts.from_interleaved(Xh, batch), X0, err_msg=f"W={W}")
        np.testing.assert_array_equal(_host(info), i0)
        assert (layouts.padding_of(Xh, batch) == SENTINEL).all()
        L = torch.full_like(Ai, SENTINEL)
        finfo = torch.empty((batch,), dtype=torch.int32, device=DEV)
        tdls.potrf_batched(Ai, layout, 0.25, out=(L, finfo), interleave=W, batch=batch)
        Lh = _host(L)
        np.testing.assert_array_equal(layouts.from_interleaved(Lh, batch), L0)
        np.testing.assert_array_equal(_host(finfo), f0)
        assert (layouts.padding_of(Lh, batch) == SENTINEL).all()
        Xs = torch.full_like(Bi, SENTINEL)
        tdls.potrs_batched(L, Bi, layout, out=Xs, interleave=W, batch=batch)
        Xsh = _host(Xs)
        np.testing.assert_array_equal(layouts.from_interleaved(Xsh, batch), X0)   # posv's bits
        assert (layouts.padding_of(Xsh, batch) == SENTINEL).all()
    Xo, io = oracle.posv(A_st, B_st, n, nrhs, layout, shift=0.25)
    assert (io == i0).all()
    ok = io == 0
    err = np.abs(X0.reshape(batch, -1)[ok] - Xo.reshape(batch, -1)[ok]).max(axis=1)
    den = np.abs(Xo.reshape(batch, -1)[ok]).max(axis=1)
    assert (err / den).max() <= 1e3 * parity.X_TOL[np.dtype(dtype)]


def test_interleaved_full_size_structure_of_arrays():
    """The headline shape as a structure of arrays (W = batch), sampled
    against the plain call."""
    w = workloads.make("n32_f64_col", seed=0, batch=65536)
    X0, p0, i0 = tdls.gesv_batched(_dev(w.A), _dev(w.B), "col")
    A = _dev(layouts.to_interleaved(w.A.reshape(w.batch, 32, 32), w.batch))
    B = _dev(layouts.to_interleaved(w.B.reshape(w.batch, 1, 32), w.batch))
    X, piv, info = tdls.gesv_batched(A, B, "col", interleave=w.batch)
    np.testing.assert_array_equal(layouts.from_interleaved(_host(X), w.batch),
                                  _host(X0).reshape(w.batch, 1, 32))
    np.testing.assert_array_equal(layouts.from_interleaved(_host(piv), w.batch), _host(p0))
    np.testing.assert_array_equal(_host(info), _host(i0))
