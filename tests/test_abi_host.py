"""The C interface on the host: the library loads, exports every declared
symbol, validates arguments and plans launches without touching a GPU.

Only validation paths that return before any device call are exercised
here: every call below either fails a scalar check, passes a null pointer,
or names overlapping buffers, so nothing is ever launched.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import dense_linear_solvers_amd as tdls

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tdls.h")


@pytest.fixture(scope="module")
def lib():
    return tdls.load_library()


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(tdls_\w+)\s*\(", text, re.M)))


def test_header_declares_the_interface():
    assert _declared_functions() == sorted(tdls.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", tdls.library_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tdls_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_strerror(lib):
    assert "gfx950" in tdls.version()
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -100, -101, -102, -103]:
        msg = tdls.strerror(code)
        assert msg and "unknown" not in msg, code
    assert "unknown" in tdls.strerror(12345)


@pytest.mark.parametrize("args,code", [
    ((7, 0, 8, 1, 1), -1),
    ((0, 5, 8, 1, 1), -2),
    ((0, 0, 0, 1, 1), -3),
    ((0, 0, 65, 1, 1), -3),
    ((0, 0, 8, 0, 1), -4),
    ((0, 0, 8, 9, 1), -4),
    ((0, 0, 8, 1, -1), -5),
])
def test_scalar_validation(lib, args, code):
    rc, _ = tdls.tdls_plan_gesv(*args)
    assert rc == code
    assert tdls.tdls_gesv_batched(*args, 0, 0, 0, 0, 0, 0) == code


def test_plan_null_out(lib):
    assert lib.tdls_plan_gesv(0, 0, 8, 1, 1, None) == -6


def test_empty_batch_launches_nothing(lib):
    # batch 0: success without looking at the pointers (all null here)
    assert tdls.tdls_gesv_batched(tdls.F64, tdls.ROW_MAJOR, 32, 1, 0, 0, 0, 0, 0, 0, 0) == 0
    p = tdls.plan_gesv("f64", "row", 32, 1, 0)
    assert p["grid"] == 0


def test_pointer_validation_before_launch(lib):
    n, nrhs, batch = 16, 2, 10
    es = 8
    a = 1 << 40                                  # never dereferenced: every call fails
    b = a + batch * n * n * es                   # before the device is queried
    x = b + batch * n * nrhs * es
    pv = x + batch * n * nrhs * es
    inf = pv + batch * n * 4
    call = lambda *ptrs: tdls.tdls_gesv_batched(tdls.F64, tdls.ROW_MAJOR, n, nrhs, batch,
                                                *ptrs, 0)
    assert call(0, b, x, pv, inf) == -6
    assert call(a + 4, b, x, pv, inf) == -6          # misaligned for float64
    assert call(a, 0, x, pv, inf) == -7
    assert call(a, b, 0, pv, inf) == -8
    assert call(a, b, a, pv, inf) == -8              # X aliases A
    assert call(a, b, b + 8, pv, inf) == -8          # X overlaps B
    assert call(a, b, x, 0, inf) == -9
    assert call(a, b, x, x + 16, inf) == -9          # piv overlaps X
    assert call(a, b, x, pv + 2, inf) == -9          # misaligned int32
    assert call(a, b, x, pv, 0) == -10
    assert call(a, b, x, pv, pv) == -10              # info overlaps piv


def test_planner_shapes(lib):
    for dtype in ("f32", "f64"):
        for n in range(1, 65):
            for nrhs in range(1, 9):
                p = tdls.plan_gesv(dtype, "row", n, nrhs, 1000)
                assert p["n_kernel"] >= n and p["nrhs_kernel"] >= nrhs
                T = p["group_size"]
                assert T & (T - 1) == 0 and 1 <= T <= 64
                assert p["rows_per_lane"] * T >= p["n_kernel"]
                assert p["systems_per_wave"] * T == 64
                assert p["systems_per_block"] * p["grid"] >= 1000
                assert (p["grid"] - 1) * p["systems_per_block"] < 1000
                assert 0 < p["lds_bytes"] <= 160 * 1024


def test_group_size_override(lib, monkeypatch):
    base = tdls.plan_gesv("f64", "col", 32, 1, 100)
    other = 64 if base["group_size"] != 64 else 16
    monkeypatch.setenv("TDLS_GROUP_SIZE", str(other))
    p = tdls.plan_gesv("f64", "col", 32, 1, 100)
    assert p["group_size"] == other
    monkeypatch.setenv("TDLS_GROUP_SIZE", "3")
    rc, _ = tdls.tdls_plan_gesv(tdls.F64, tdls.COL_MAJOR, 32, 1, 100)
    assert rc == -103


@pytest.mark.parametrize("args,code", [
    ((7, 0, 8, 1), -1),
    ((0, 5, 8, 1), -2),
    ((0, 0, 0, 1), -3),
    ((0, 0, 65, 1), -3),
    ((0, 0, 8, -1), -4),
])
def test_getrf_scalar_validation(lib, args, code):
    assert tdls.tdls_getrf_batched(*args, 0, 0, 0, 0, 0) == code


@pytest.mark.parametrize("args,code", [
    ((7, 0, 8, 1, 1), -1),
    ((0, 5, 8, 1, 1), -2),
    ((0, 0, 0, 1, 1), -3),
    ((0, 0, 8, 0, 1), -4),
    ((0, 0, 8, 9, 1), -4),
    ((0, 0, 8, 1, -1), -5),
])
def test_getrs_scalar_validation(lib, args, code):
    assert tdls.tdls_getrs_batched(*args, 0, 0, 0, 0, 0) == code


def test_plan_op_validation_and_shapes(lib):
    assert tdls.tdls_plan_op(9, 0, 0, 8, 1, 1)[0] == -1
    assert tdls.tdls_plan_op(tdls.OP_GETRS, 7, 0, 8, 1, 1)[0] == -2
    assert tdls.tdls_plan_op(tdls.OP_GETRS, 0, 0, 8, 9, 1)[0] == -5
    assert tdls.tdls_plan_op(tdls.OP_GETRF, 0, 0, 8, 99, 1)[0] == 0   # nrhs ignored
    assert tdls.tdls_plan_op(tdls.OP_GETRF, 0, 0, 8, 1, -1)[0] == -6
    assert lib.tdls_plan_op(0, 0, 0, 8, 1, 1, None) == -7
    for dtype in ("f32", "f64"):
        for n in (1, 8, 13, 32, 64):
            g = tdls.plan_gesv(dtype, "row", n, 1, 1000)
            f = tdls.plan_op("getrf", dtype, "row", n, 1, 1000)
            assert f["group_size"] == g["group_size"] and f["lds_bytes"] == g["lds_bytes"]
            for nrhs in (1, 3, 8):
                s = tdls.plan_op("getrs", dtype, "col", n, nrhs, 1000)
                N, R = s["n_kernel"], s["nrhs_kernel"]
                es = 8 if dtype == "f64" else 4
                vec = 16 // es
                tri = max(-(-(N * (N + 1) // 2) // vec) * vec, N * R)
                elems = -(-tri // vec) * vec if R >= 4 else 0
                stage = -(-(N * R * es) // 16) * 16 if (R < 4 and s["group_size"] >= 16) else 0
                per_group = -(-(N * 4) // 16) * 16 + elems * es + stage
                assert s["lds_bytes"] == s["systems_per_wave"] * per_group
                assert s["systems_per_block"] * s["grid"] >= 1000


def test_factor_solve_pointer_validation(lib):
    n, nrhs, batch = 16, 2, 10
    es = 8
    a = 1 << 40                                  # never dereferenced: every call fails
    lu = a + batch * n * n * es                  # before the device is queried
    pv = lu + batch * n * n * es
    inf = pv + batch * n * 4
    b = inf + batch * 4 + 64
    x = b + batch * n * nrhs * es
    f = lambda *p: tdls.tdls_getrf_batched(tdls.F64, tdls.COL_MAJOR, n, batch, *p, 0)
    assert f(0, lu, pv, inf) == -5
    assert f(a, 0, pv, inf) == -6
    assert f(a, a + 8, pv, inf) == -6            # LU overlaps A
    assert f(a, lu, 0, inf) == -7
    assert f(a, lu, lu + 8, inf) == -7           # piv overlaps LU
    assert f(a, lu, pv, 0) == -8
    assert f(a, lu, pv, pv + 4) == -8            # info overlaps piv
    s = lambda *p: tdls.tdls_getrs_batched(tdls.F64, tdls.COL_MAJOR, n, nrhs, batch, *p, 0)
    assert s(0, pv, b, x) == -6
    assert s(lu, 0, b, x) == -7
    assert s(lu, pv + 2, b, x) == -7             # misaligned int32
    assert s(lu, pv, 0, x) == -8
    assert s(lu, pv, b, 0) == -9
    assert s(lu, pv, b, b) == -9                 # X aliases B
    assert s(lu, pv, b, lu) == -9                # X overlaps LU
    assert tdls.tdls_getrf_batched(tdls.F64, tdls.ROW_MAJOR, n, 0, 0, 0, 0, 0, 0) == 0
    assert tdls.tdls_getrs_batched(tdls.F64, tdls.ROW_MAJOR, n, 1, 0, 0, 0, 0, 0, 0) == 0


def test_cholesky_validation_before_launch(lib):
    n, nrhs, batch = 16, 2, 10
    es = 8
    a = 1 << 40                                  # never dereferenced: every call fails
    l = a + batch * n * n * es                   # before the device is queried
    inf = l + batch * n * n * es
    b = inf + batch * 4 + 64
    x = b + batch * n * nrhs * es
    assert tdls.tdls_potrf_batched(7, 0, n, batch, 0.0, a, l, inf, 0) == -1
    assert tdls.tdls_potrf_batched(0, 0, 65, batch, 0.0, a, l, inf, 0) == -3
    assert tdls.tdls_potrf_batched(0, 0, n, -1, 0.0, a, l, inf, 0) == -4
    f = lambda shift, *p: tdls.tdls_potrf_batched(tdls.F64, tdls.ROW_MAJOR, n, batch, shift, *p, 0)
    assert f(float("nan"), a, l, inf) == -5
    assert f(0.0, 0, l, inf) == -6
    assert f(0.0, a, a, inf) == -7
    assert f(0.0, a, l, l) == -8
    s = lambda shift, *p: tdls.tdls_posv_batched(tdls.F64, tdls.COL_MAJOR, n, nrhs, batch, shift,
                                                 *p, 0)
    assert tdls.tdls_posv_batched(0, 0, n, 0, batch, 0.0, a, b, x, inf, 0) == -4
    assert tdls.tdls_posv_batched(0, 0, n, 1, -1, 0.0, a, b, x, inf, 0) == -5
    assert s(float("-inf"), a, b, x, inf) == -6
    assert s(0.0, 0, b, x, inf) == -7
    assert s(0.0, a, 0, x, inf) == -8
    assert s(0.0, a, b, a, inf) == -9
    assert s(0.0, a, b, x, x) == -10
    assert tdls.tdls_posv_batched(tdls.F64, tdls.ROW_MAJOR, n, 1, 0, 0.0, 0, 0, 0, 0, 0) == 0
    p = tdls.plan_op("posv", "f64", "col", 32, 1, 1000)
    ch = min(p["group_size"], 16)       # symmetry chunk rows, stride n + 1
    per_group = max(ch * 33, 32 * 33 // 2, 32 * 1)
    assert p["lds_bytes"] == p["systems_per_wave"] * per_group * 8
    assert tdls.plan_op("potrf", "f32", "row", 13, 5, 10)["nrhs_kernel"] == 1


def test_options_validation_before_launch(lib):
    n, nrhs, batch = 16, 2, 10
    es = 8
    a = 1 << 40                                  # never dereferenced: every call fails
    b = a + batch * n * n * es                   # before the device is queried
    x = b + batch * n * nrhs * es
    pv = x + batch * n * nrhs * es
    inf = pv + batch * n * 4
    Opt = tdls.Options
    g = lambda opt, *p: tdls.tdls_gesv_batched_ex(tdls.F64, tdls.ROW_MAJOR, n, nrhs, batch, opt,
                                                  *p, 0)
    # scalar arguments first, then the options, then the pointers (shifted by one)
    assert tdls.tdls_gesv_batched_ex(9, 0, n, nrhs, batch, None, a, b, x, pv, inf, 0) == -1
    assert tdls.tdls_gesv_batched_ex(1, 0, n, nrhs, -2, Opt(8, 0, 1), a, b, x, pv, inf, 0) == -5
    assert g(Opt(2, 0, 1), a, b, x, pv, inf) == -6      # unknown flag
    assert g(Opt(1, 7, 1), a, b, x, pv, inf) == -6      # reserved field
    assert g(Opt(1, 0, 11), a, b, x, pv, inf) == -6     # interleave above batch
    assert g(Opt(1, 0, -1), a, b, x, pv, inf) == -6
    assert g(None, 0, b, x, pv, inf) == -7
    assert g(Opt(1, 0, 0), a, 0, x, pv, inf) == -8
    assert g(Opt(1, 0, 1), a, b, a, pv, inf) == -9
    assert g(Opt(1, 0, 1), a, b, x, x, inf) == -10
    assert g(Opt(1, 0, 1), a, b, x, pv, pv) == -11
    assert tdls.tdls_gesv_batched_ex(1, 0, n, nrhs, 0, Opt(1, 0, 1), 0, 0, 0, 0, 0, 0) == 0
    f = lambda opt, *p: tdls.tdls_getrf_batched_ex(tdls.F64, tdls.COL_MAJOR, n, batch, opt, *p, 0)
    lu = a + batch * n * n * es
    pv = lu + batch * n * n * es
    inf = pv + batch * n * 4
    assert tdls.tdls_getrf_batched_ex(1, 0, n, -1, None, a, lu, pv, inf, 0) == -4
    assert f(Opt(3, 0, 1), a, lu, pv, inf) == -5
    assert f(Opt(1, 0, 1), 0, lu, pv, inf) == -6
    assert f(Opt(1, 0, 1), a, a, pv, inf) == -7
    assert f(None, a, lu, 0, inf) == -8
    assert f(None, a, lu, pv, pv) == -9
    for code in (-11,):
        assert "unknown" not in tdls.strerror(code)


def test_interleaved_spans_and_ex_numbering(lib):
    """Under interleave W the buffers span whole blocks of W systems, so a
    buffer that starts right after batch systems overlaps; the *_ex calls
    number their pointer arguments after the options argument."""
    n, nrhs, batch, W = 8, 1, 10, 4                 # 3 blocks: 12 systems spanned
    es = 8
    Opt = tdls.Options
    a = 1 << 40
    tight = a + batch * n * n * es                   # fine for W = 1, overlaps for W = 4
    roomy = a + 12 * n * n * es
    x = roomy + 12 * n * n * es
    pv = x + 12 * n * nrhs * es
    inf = pv + 12 * n * 4
    f = lambda opt, lu: tdls.tdls_getrf_batched_ex(tdls.F64, tdls.ROW_MAJOR, n, batch, opt, a,
                                                   lu, pv, inf, 0)
    assert f(Opt(0, 0, W), tight) == -7
    assert f(Opt(0, 0, 0), 0) == -7
    # getrs_ex: [6] opt (no flags), [7] LU, [8] piv, [9] B, [10] X
    r = lambda opt, *p: tdls.tdls_getrs_batched_ex(tdls.F64, tdls.COL_MAJOR, n, nrhs, batch, opt,
                                                   *p, 0)
    assert r(Opt(1, 0, W), a, pv, x, roomy) == -6        # scaling is not a getrs option
    assert r(Opt(0, 0, batch + 1), a, pv, x, roomy) == -6
    assert r(Opt(0, 0, W), 0, pv, x, roomy) == -7
    assert r(Opt(0, 0, W), a, 0, x, roomy) == -8
    assert r(Opt(0, 0, W), a, pv, 0, roomy) == -9
    assert r(Opt(0, 0, W), a, pv, x, tight) == -10       # X overlaps LU's span
    # potrf_ex: [5] shift, [6] opt, [7] A, [8] L, [9] info
    c = lambda shift, opt, *p: tdls.tdls_potrf_batched_ex(tdls.F64, tdls.ROW_MAJOR, n, batch,
                                                          shift, opt, *p, 0)
    assert tdls.tdls_potrf_batched_ex(0, 0, n, -1, 0.0, None, a, roomy, inf, 0) == -4
    assert c(float("inf"), None, a, roomy, inf) == -5
    assert c(0.0, Opt(1, 0, 1), a, roomy, inf) == -6
    assert c(0.0, Opt(0, 0, W), 0, roomy, inf) == -7
    assert c(0.0, Opt(0, 0, W), a, tight, inf) == -8
    assert c(0.0, Opt(0, 0, W), a, roomy, 0) == -9
    # posv_ex: [6] shift, [7] opt, [8] A, [9] B, [10] X, [11] info
    v = lambda shift, opt, *p: tdls.tdls_posv_batched_ex(tdls.F64, tdls.ROW_MAJOR, n, nrhs, batch,
                                                         shift, opt, *p, 0)
    assert v(float("nan"), None, a, roomy, x, inf) == -6
    assert v(0.0, Opt(0, 3, 1), a, roomy, x, inf) == -7
    assert v(0.0, Opt(0, 0, W), 0, roomy, x, inf) == -8
    assert v(0.0, Opt(0, 0, W), a, 0, x, inf) == -9
    assert v(0.0, Opt(0, 0, W), a, roomy, a, inf) == -10
    assert v(0.0, Opt(0, 0, W), a, roomy, x, 0) == -11
    # an empty batch launches nothing, whatever the interleave
    assert tdls.tdls_posv_batched_ex(1, 0, n, 1, 0, 0.0, Opt(0, 0, 9), 0, 0, 0, 0, 0) == 0


def test_potrs_validation_before_launch(lib):
    n, nrhs, batch = 16, 2, 10
    es = 8
    l = 1 << 40                                  # never dereferenced: every call fails
    b = l + batch * n * n * es                   # before the device is queried
    x = b + batch * n * nrhs * es
    f = lambda *p: tdls.tdls_potrs_batched(tdls.F64, tdls.ROW_MAJOR, n, nrhs, batch, *p, 0)
    assert tdls.tdls_potrs_batched(5, 0, n, nrhs, batch, l, b, x, 0) == -1
    assert tdls.tdls_potrs_batched(0, 0, n, 9, batch, l, b, x, 0) == -4
    assert tdls.tdls_potrs_batched(0, 0, n, 1, 0, 0, 0, 0, 0) == 0     # empty batch
    assert f(0, b, x) == -6
    assert f(l + 4, b, x) == -6
    assert f(l, 0, x) == -7
    assert f(l, b, l) == -8                      # X overlaps L
    assert f(l, b, b + 8) == -8                  # X overlaps B
    Opt = tdls.Options
    g = lambda opt, *p: tdls.tdls_potrs_batched_ex(tdls.F64, tdls.COL_MAJOR, n, nrhs, batch, opt,
                                                   *p, 0)
    assert g(Opt(1, 0, 1), l, b, x) == -6        # no scaling option for potrs
    assert g(Opt(0, 0, 4), 0, b, x) == -7
    assert g(Opt(0, 0, 4), l, b, l) == -9
    p = tdls.plan_op("potrs", "f64", "row", 32, 3, 1000)
    assert p == tdls.plan_op("posv", "f64", "row", 32, 3, 1000)


def test_group_size_choice_per_op(lib):
    """LU in float64 at n = 16 runs 16-lane groups at every batch size; the
    Cholesky kernels and float32 keep 4-lane groups there (large batches),
    and float32 takes them up to n = 24 where the rows fit."""
    big = 1 << 20
    for n in (9, 16):
        for op in ("getrf", "getrs"):
            assert tdls.plan_op(op, "f64", "row", n, 1, big)["group_size"] == 16
        assert tdls.plan_gesv("f64", "row", n, 4, big)["group_size"] == 16
        for op in ("potrf", "posv", "potrs"):
            assert tdls.plan_op(op, "f64", "row", n, 1, big)["group_size"] == 4
        assert tdls.plan_gesv("f32", "row", n, 4, big)["group_size"] == 4
    assert tdls.plan_gesv("f64", "row", 8, 1, big)["group_size"] == 4
    # float32 at n = 17..24: quads where six rows per lane fit (one or two
    # right-hand sides), except getrs; 16-lane groups with more right-hand sides
    for n in (17, 24):
        for nrhs in (1, 2):
            assert tdls.plan_gesv("f32", "row", n, nrhs, big)["group_size"] == 4
            for op in ("posv", "potrs"):
                assert tdls.plan_op(op, "f32", "row", n, nrhs, big)["group_size"] == 4
            assert tdls.plan_op("getrs", "f32", "row", n, nrhs, big)["group_size"] == 16
        for op in ("getrf", "potrf"):
            assert tdls.plan_op(op, "f32", "row", n, 1, big)["group_size"] == 4
        assert tdls.plan_gesv("f32", "row", n, 4, big)["group_size"] == 16
        assert tdls.plan_gesv("f64", "row", n, 1, big)["group_size"] == 16


def test_out_tensors_are_checked_before_any_call():
    """``out=`` tensors must be exactly what the call would allocate (the C
    layer sees raw pointers only); a mismatch raises before the library is
    called.  Checked on CPU tensors against a CPU device."""
    import torch
    from dense_linear_solvers_amd import _binding as b
    dev = torch.device("cpu")
    good = torch.empty((4, 16, 2), dtype=torch.float64)
    b._check_out(torch, good, "X", torch.float64, dev, (4, 16, 2))
    with pytest.raises(TypeError):
        b._check_out(torch, good.float(), "X", torch.float64, dev, (4, 16, 2))
    with pytest.raises(ValueError):
        b._check_out(torch, good[:3], "X", torch.float64, dev, (4, 16, 2))
    with pytest.raises(ValueError):
        b._check_out(torch, good.transpose(1, 2), "X", torch.float64, dev, (4, 2, 16))
    with pytest.raises(ValueError):
        b._check_out(torch, good, "X", torch.float64, torch.device("meta"), (4, 16, 2))
    with pytest.raises(TypeError):
        b._check_out(torch, good.numpy(), "X", torch.float64, dev, (4, 16, 2))
    piv = torch.empty((4, 16), dtype=torch.int64)
    with pytest.raises(TypeError):
        b._check_out(torch, piv, "piv", torch.int32, dev, (4, 16))
    with pytest.raises(TypeError):
        b._unpack_out((good, piv), ("X", "piv", "info"))
    assert b._unpack_out(good, ("X",)) == (good,)
