"""GPU parity: the HIP library through its C interface vs the CPU oracle.

Every test here needs an MI355X and the built library (marker ``gpu``).
Inputs are the seeded recipes of dense_linear_solvers_amd.workloads (small
batches spanning several blocks and a ragged tail, then the full sizes with
sampled oracle checks) plus hand-built and edge cases.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import golden_io
import metrics
import oracle
import parity
import dense_linear_solvers_amd as tdls
from dense_linear_solvers_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(dt):
    return np.float32 if dt == "f32" else np.float64


def run_gpu(A_st: np.ndarray, B_st: np.ndarray, layout: str):
    """Upload storage arrays, solve, return host copies (X_st, piv, info)."""
    A = torch.from_numpy(np.ascontiguousarray(A_st)).to(DEV)
    B = torch.from_numpy(np.ascontiguousarray(B_st)).to(DEV)
    X, piv, info = tdls.gesv_batched(A, B, layout)
    torch.cuda.synchronize()
    return X.cpu().numpy(), piv.cpu().numpy(), info.cpu().numpy()


def assert_parity(rep: parity.Report, what: str):
    print(f"{what}: {rep}", flush=True)
    assert rep.info_mismatch == 0, what
    assert rep.piv_mismatch_margin == 0, what
    assert rep.failed_bad_outputs == 0, what
    assert rep.x_max_err <= rep.x_tol, what
    assert rep.resid_max <= parity.RESID_TOL, what


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tdls.load_library()
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------- hand-worked


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [3, 8, 24, 64])
def test_golden_examples(dtype, layout, n):
    for ex in golden_io.all_examples():
        e = golden_io.embed_identity(ex, n) if n > 3 else ex
        A = e["A"][None].astype(_np(dtype))
        b = e["b"][None, :, None].astype(_np(dtype))
        X, piv, info = run_gpu(oracle.to_storage(A, layout), oracle.rhs_to_storage(b, layout),
                               layout)
        X = oracle.rhs_from_storage(X, layout, n, 1)
        assert info[0] == e["info"], (e["name"], n)
        np.testing.assert_array_equal(piv[0], e["piv"], err_msg=e["name"])
        np.testing.assert_array_equal(X[0, :, 0], e["x"].astype(_np(dtype)), err_msg=e["name"])
        if e["info"] != 0:
            assert not np.signbit(X).any()


# ----------------------------------------------- recipes, oracle-sized


RECIPE_NAMES = sorted(workloads.RECIPES)


@pytest.mark.parametrize("name", RECIPE_NAMES)
def test_recipe_parity_small(name):
    """Every recipe at a batch that spans many blocks and ends ragged."""
    r = workloads.RECIPES[name]
    plan = tdls.plan_gesv(r.dtype, r.layout, r.n, r.nrhs, 1)
    batch = 37 * plan["systems_per_block"] + 5
    w = workloads.make(name, seed=0, batch=batch, gap_fn=oracle.pivot_gap)
    X, piv, info = run_gpu(w.A, w.B, w.layout)
    rep = parity.compare(w.A, w.B, X, piv, info, w.n, w.nrhs, w.layout)
    assert_parity(rep, f"{name} batch={batch}")
    if name == "n16_f32_row_sing":
        assert (info[w.meta["singular"]] == 16).all()


# ------------------------------------------------- recipes, full size


@pytest.mark.parametrize("name", RECIPE_NAMES)
def test_recipe_parity_full_size(name):
    """Full-size batch in the benchmark's launch configuration, every
    system compared with the oracle (in chunks); every system is also
    checked for a finite solution or a valid failure record."""
    w = workloads.make(name, seed=0, gap_fn=oracle.pivot_gap if name == "n32_f64_col" else None)
    X, piv, info = run_gpu(w.A, w.B, w.layout)
    rep = parity.compare_chunked(w.A, w.B, X, piv, info, w.n, w.nrhs, w.layout)
    assert rep.systems == w.batch
    assert_parity(rep, f"{name} full batch={w.batch}, every system")
    Xf = X.reshape(w.batch, -1)
    ok = info == 0
    assert np.isfinite(Xf[ok]).all()
    assert ((piv[ok] >= np.arange(w.n)) & (piv[ok] < w.n)).all()
    assert (Xf[~ok] == 0).all() and (piv[~ok] == -1).all()
    if name == "n16_f32_row_sing":
        assert (info[w.meta["singular"]] == 16).all()
        others = np.setdiff1d(np.arange(w.batch), w.meta["singular"])
        assert (info[others] == 0).all()


# ------------------------------------------------------ every shape


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_every_n_and_nrhs(dtype, layout):
    """n = 1..64 and nrhs = 1..8 (padded kernels included), small ragged batch."""
    rng = np.random.default_rng(99)
    for n in range(1, 65):
        nrhs = int(rng.integers(1, 9))
        batch = int(rng.integers(1, 40))
        A = rng.standard_normal((batch, n, n)) + 0.5 * np.eye(n)
        B = rng.standard_normal((batch, n, nrhs))
        A_st = oracle.to_storage(A.astype(_np(dtype)), layout)
        B_st = oracle.rhs_to_storage(B.astype(_np(dtype)), layout)
        X, piv, info = run_gpu(A_st, B_st, layout)
        rep = parity.compare(A_st, B_st, X, piv, info, n, nrhs, layout)
        assert_parity(rep, f"{dtype} {layout} n={n} nrhs={nrhs} batch={batch}")


# --------------------------------------------------- singular systems


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("n", [8, 16, 24, 32, 64])
def test_singular_constructions(dtype, n):
    rng = np.random.default_rng(5 + n)
    batch = 300
    A = rng.uniform(-1, 1, (batch, n, n)).astype(_np(dtype))
    kind = np.arange(batch) % 4
    expect = np.zeros(batch, np.int32)
    for s in range(batch):
        if kind[s] == 1:          # duplicated row -> n
            i, k = rng.choice(n, size=2, replace=False)
            A[s, k] = A[s, i]
            expect[s] = n
        elif kind[s] == 2:        # zero column j -> j + 1
            j = int(rng.integers(0, n))
            A[s, :, j] = 0
            expect[s] = j + 1
        elif kind[s] == 3 and s % 8 == 3:   # zero matrix -> 1
            A[s] = 0
            expect[s] = 1
    B = rng.uniform(-1, 1, (batch, n, 2)).astype(_np(dtype))
    X, piv, info = run_gpu(A, B, "row")
    np.testing.assert_array_equal(info, expect)
    rep = parity.compare(A, B, X, piv, info, n, 2, "row")
    assert_parity(rep, f"singular {dtype} n={n}")


# ------------------------------------------------------- invariances


def _built_group_sizes(monkeypatch, dtype, n, nrhs):
    """Group sizes the library has kernels for at this shape."""
    sizes = []
    for t in (1, 2, 4, 8, 16, 32, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_gesv(tdls.F64 if dtype == "f64" else tdls.F32, tdls.ROW_MAJOR,
                                    n, nrhs, 1)
        if rc == 0:
            sizes.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return sizes


def test_group_size_does_not_change_results(monkeypatch):
    """Results are bit-identical for every group size built for a shape."""
    rng = np.random.default_rng(42)
    compared = 0
    for dtype in ("f32", "f64"):
        # kernel sizes, and ragged sizes run by a larger kernel (phantom rows
        # in the last slot, across the slot boundaries where rows are put
        # back in position order)
        for n in (5, 8, 13, 16, 20, 24, 30, 32):
            for nrhs in (1, 2, 4, 8):
                sizes = _built_group_sizes(monkeypatch, dtype, n, nrhs)
                if len(sizes) < 2:
                    continue
                A = rng.standard_normal((301, n, n)).astype(_np(dtype))
                B = rng.standard_normal((301, n, nrhs)).astype(_np(dtype))
                A[7, 3] = A[7, 1]
                results = []
                for t in sizes:
                    monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
                    results.append(run_gpu(A, B, "row"))
                monkeypatch.delenv("TDLS_GROUP_SIZE")
                for t, r in zip(sizes[1:], results[1:]):
                    for u, v in zip(results[0], r):
                        np.testing.assert_array_equal(
                            u, v, err_msg=f"{dtype} n={n} nrhs={nrhs} T={sizes[0]}/{t}")
                compared += 1
    assert compared > 0


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_layouts_give_identical_bits(dtype):
    rng = np.random.default_rng(8)
    for n, nrhs in ((8, 1), (16, 4), (24, 2), (32, 1), (64, 8)):
        A = rng.standard_normal((129, n, n)).astype(_np(dtype))
        B = rng.standard_normal((129, n, nrhs)).astype(_np(dtype))
        Xr, pr, ir = run_gpu(oracle.to_storage(A, "row"), oracle.rhs_to_storage(B, "row"), "row")
        Xc, pc, ic = run_gpu(oracle.to_storage(A, "col"), oracle.rhs_to_storage(B, "col"), "col")
        np.testing.assert_array_equal(Xr, oracle.rhs_from_storage(Xc, "col", n, nrhs))
        np.testing.assert_array_equal(pr, pc)
        np.testing.assert_array_equal(ir, ic)


# ---------------------------------------------------------- contract


def test_inputs_are_read_only_and_outputs_fully_written():
    rng = np.random.default_rng(3)
    A = torch.from_numpy(rng.standard_normal((1000, 32, 32))).to(DEV)
    B = torch.from_numpy(rng.standard_normal((1000, 32, 1))).to(DEV)
    A0, B0 = A.clone(), B.clone()
    X = torch.full_like(B, float("nan"))
    piv = torch.full((1000, 32), -7, dtype=torch.int32, device=DEV)
    info = torch.full((1000,), -7, dtype=torch.int32, device=DEV)
    tdls.gesv_batched(A, B, "row", out=(X, piv, info))
    torch.cuda.synchronize()
    assert torch.equal(A, A0) and torch.equal(B, B0)
    assert torch.isfinite(X).all() and (piv >= 0).all() and (info == 0).all()


def test_empty_batch_and_argument_errors():
    A = torch.zeros((0, 16, 16), dtype=torch.float32, device=DEV)
    B = torch.zeros((0, 16, 2), dtype=torch.float32, device=DEV)
    X, piv, info = tdls.gesv_batched(A, B, "row")
    assert X.shape == (0, 16, 2) and piv.shape == (0, 16) and info.shape == (0,)
    A = torch.randn((4, 16, 16), device=DEV)
    B = torch.randn((4, 16, 2), device=DEV)
    piv = torch.empty((4, 16), dtype=torch.int32, device=DEV)
    info = torch.empty((4,), dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    rc = tdls.tdls_gesv_batched(tdls.F32, tdls.ROW_MAJOR, 16, 2, 4, A.data_ptr(), B.data_ptr(),
                                A.data_ptr(), piv.data_ptr(), info.data_ptr(), s)
    assert rc == -8                       # X aliases A: rejected, nothing launched
    torch.cuda.synchronize()


def test_non_default_stream_and_batch_edges():
    rng = np.random.default_rng(10)
    st = torch.cuda.Stream()
    for n, nrhs, dtype in ((16, 4, "f32"), (32, 1, "f64"), (64, 8, "f64")):
        spb = tdls.plan_gesv(dtype, "row", n, nrhs, 1)["systems_per_block"]
        for batch in (1, spb - 1, spb, spb + 1):
            if batch < 1:
                continue
            A_np = rng.standard_normal((batch, n, n)).astype(_np(dtype))
            B_np = rng.standard_normal((batch, n, nrhs)).astype(_np(dtype))
            with torch.cuda.stream(st):
                A = torch.from_numpy(A_np).to(DEV, non_blocking=False)
                B = torch.from_numpy(B_np).to(DEV, non_blocking=False)
                X, piv, info = tdls.gesv_batched(A, B, "row", stream=st)
            st.synchronize()
            rep = parity.compare(A_np, B_np, X.cpu().numpy(), piv.cpu().numpy(),
                                 info.cpu().numpy(), n, nrhs, "row")
            assert_parity(rep, f"stream n={n} batch={batch}")
