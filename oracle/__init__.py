"""CPU oracle for batched gesv (LU with partial row pivoting + solve).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain reference that the GPU
library is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library never does, and
the oracle never imports the library.

The arithmetic lives in ``gesv_oracle.c`` (plain C, one system at a time,
working precision, explicit fma, correctly rounded division); this module only
marshals numpy arrays to it.  Citations of the pages for each step are in the C
source.

Storage convention (shared with the library's boundary, restated here):
  * ``layout="row"``: A of system s is row-major, element (r, c) at r*n + c;
    B and X are n x nrhs row-major, (r, j) at r*nrhs + j.
  * ``layout="col"``: A is column-major, (r, c) at c*n + r; B and X are
    column-major, (r, j) at j*n + r.
Systems are contiguous: system s starts at s*n*n in A, s*n*nrhs in B and X,
s*n in piv and s in info.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build, library_path

__all__ = ["gesv", "getrf", "getrs", "potrf", "potrs", "posv", "pivot_gap", "build", "library_path", "to_storage", "from_storage",
           "rhs_to_storage", "rhs_from_storage", "max_threads", "use_library"]

_LAYOUTS = {"row": 0, "col": 1}
_libs: dict = {}
# TDLS_ORACLE_LIB: load another build of the oracle (the sanitized one)
_active_path = os.environ.get("TDLS_ORACLE_LIB") or None


def _load():
    path = _active_path or library_path()
    lib = _libs.get(path)
    if lib is None:
        if path == library_path() and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int32)
        for sfx, ct in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
            tp = ctypes.POINTER(ct)
            g = getattr(lib, "oracle_gesv_" + sfx)
            g.restype = ctypes.c_int
            g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                          ctypes.c_int, tp, tp, tp, i32p, i32p, ctypes.c_int]
            r = getattr(lib, "oracle_getrs_" + sfx)
            r.restype = ctypes.c_int
            r.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                          tp, i32p, tp, tp, ctypes.c_int]
            c = getattr(lib, "oracle_potrf_" + sfx)
            c.restype = ctypes.c_int
            c.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_double, tp, tp,
                          i32p, ctypes.c_int]
            t = getattr(lib, "oracle_potrs_" + sfx)
            t.restype = ctypes.c_int
            t.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, tp, tp, tp,
                          ctypes.c_int]
            v = getattr(lib, "oracle_posv_" + sfx)
            v.restype = ctypes.c_int
            v.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                          ctypes.c_double, tp, tp, tp, i32p, ctypes.c_int]
            f = getattr(lib, "oracle_getrf_" + sfx)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, tp, tp, i32p,
                          i32p, ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        _libs[path] = lib
    return lib


class use_library:
    """Context manager: route the functions of this module to another build
    of the oracle source (the tests use it to run the pins against copies of
    the oracle with a deliberately planted mistake)."""

    def __init__(self, path: str):
        self.path = path
        self.prev = None

    def __enter__(self):
        global _active_path
        self.prev = _active_path
        _active_path = self.path
        return self

    def __exit__(self, *exc):
        global _active_path
        _active_path = self.prev
        return False


def max_threads() -> int:
    """Threads the oracle's OpenMP runtime would use by default."""
    return int(_load().oracle_max_threads())


def _sfx(dtype):
    dt = np.dtype(dtype)
    if dt == np.float64:
        return "f64", ctypes.c_double
    if dt == np.float32:
        return "f32", ctypes.c_float
    raise TypeError(f"oracle supports float32 and float64, not {dt}")


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def to_storage(A_logical: np.ndarray, layout: str) -> np.ndarray:
    """Logical matrices [batch, n, n] -> contiguous storage in ``layout``."""
    A_logical = np.asarray(A_logical)
    if layout == "row":
        return np.ascontiguousarray(A_logical)
    return np.ascontiguousarray(A_logical.transpose(0, 2, 1))


def from_storage(A_store: np.ndarray, layout: str, n: int) -> np.ndarray:
    """Contiguous storage -> logical matrices [batch, n, n]."""
    A = np.asarray(A_store).reshape(-1, n, n)
    return A if layout == "row" else A.transpose(0, 2, 1)


def rhs_to_storage(B_logical: np.ndarray, layout: str) -> np.ndarray:
    """Logical right-hand sides [batch, n, nrhs] -> contiguous storage."""
    B_logical = np.asarray(B_logical)
    if layout == "row":
        return np.ascontiguousarray(B_logical)
    return np.ascontiguousarray(B_logical.transpose(0, 2, 1))


def rhs_from_storage(B_store: np.ndarray, layout: str, n: int, nrhs: int) -> np.ndarray:
    """Contiguous storage -> logical right-hand sides [batch, n, nrhs]."""
    if layout == "row":
        return np.asarray(B_store).reshape(-1, n, nrhs)
    return np.asarray(B_store).reshape(-1, nrhs, n).transpose(0, 2, 1)


def gesv(A_store: np.ndarray, B_store: np.ndarray, n: int, nrhs: int, layout: str = "row",
         nthreads: int = 0, scale: bool = False):
    """Solve every system of a batch.

    ``A_store`` / ``B_store`` are the raw contiguous storage of the batch (any
    shape with batch*n*n / batch*n*nrhs elements, float32 or float64, same
    dtype).  Returns ``(X_store, piv, info)``: X in B's storage, piv int32
    [batch, n] (0-based swap sequence, all -1 for a failed system), info int32
    [batch]: 0; -1 for a non-finite entry of A or B; k >= 1, the 1-based step
    of the first exactly zero pivot; -3 for a non-finite computed value.
    ``scale`` divides each system by the largest magnitude of its matrix
    first (the whole-matrix max-abs scaling).
    """
    sfx, ct = _sfx(A_store.dtype)
    if np.dtype(B_store.dtype) != np.dtype(A_store.dtype):
        raise TypeError("A and B must share a dtype")
    A = np.ascontiguousarray(A_store).reshape(-1)
    B = np.ascontiguousarray(B_store).reshape(-1)
    if A.size % (n * n) != 0:
        raise ValueError("A size is not a multiple of n*n")
    batch = A.size // (n * n)
    if B.size != batch * n * nrhs:
        raise ValueError("B size does not match batch*n*nrhs")
    X = np.empty_like(B)
    piv = np.empty((batch, n), dtype=np.int32)
    info = np.empty((batch,), dtype=np.int32)
    rc = getattr(_load(), "oracle_gesv_" + sfx)(
        _LAYOUTS[layout], n, nrhs, batch, int(bool(scale)), _ptr(A, ct), _ptr(B, ct),
        _ptr(X, ct), _ptr(piv, ctypes.c_int32), _ptr(info, ctypes.c_int32), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gesv_{sfx} returned {rc}")
    return X.reshape(np.shape(B_store)), piv, info


def getrf(A_store: np.ndarray, n: int, layout: str = "row", nthreads: int = 0,
          scale: bool = False):
    """Factor every matrix of a batch, without stopping at a zero pivot.

    Returns ``(LU, ipiv, info, gap)``: LU float [batch, n, n] logical row-major
    (unit-lower L below the diagonal, U on and above it, LAPACK row order),
    ipiv int32 [batch, n] (0-based swap sequence), info int32 [batch] (as for
    ``gesv``) and gap float64 [batch], the smallest relative distance between
    the two largest candidate magnitudes over steps 0..n-2.  The factors of a
    failed system are returned as computed (all +0.0 with ipiv -1 for status
    -1).  ``scale``: max-abs scaling, U multiplied back at the end.
    """
    sfx, ct = _sfx(A_store.dtype)
    A = np.ascontiguousarray(A_store).reshape(-1)
    if A.size % (n * n) != 0:
        raise ValueError("A size is not a multiple of n*n")
    batch = A.size // (n * n)
    LU = np.empty((batch, n, n), dtype=A.dtype)
    ipiv = np.empty((batch, n), dtype=np.int32)
    info = np.empty((batch,), dtype=np.int32)
    gap = np.empty((batch,), dtype=np.float64)
    rc = getattr(_load(), "oracle_getrf_" + sfx)(
        _LAYOUTS[layout], n, batch, int(bool(scale)), _ptr(A, ct), _ptr(LU, ct),
        _ptr(ipiv, ctypes.c_int32), _ptr(info, ctypes.c_int32), _ptr(gap, ctypes.c_double),
        int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_getrf_{sfx} returned {rc}")
    return LU, ipiv, info, gap


def getrs(LU_store: np.ndarray, ipiv: np.ndarray, B_store: np.ndarray, n: int, nrhs: int,
          layout: str = "row", nthreads: int = 0) -> np.ndarray:
    """Solve from factors: ``LU_store`` is the storage (in ``layout``) of the
    factors in LAPACK's row order (see ``getrf``; convert its logical output
    with ``to_storage``), ``ipiv`` int32 [batch, n] the 0-based swap sequence
    (a system whose first entry is negative gets X = +0.0), ``B_store`` the
    right-hand sides.  Returns X in B's storage."""
    sfx, ct = _sfx(LU_store.dtype)
    if np.dtype(B_store.dtype) != np.dtype(LU_store.dtype):
        raise TypeError("LU and B must share a dtype")
    LU = np.ascontiguousarray(LU_store).reshape(-1)
    B = np.ascontiguousarray(B_store).reshape(-1)
    P = np.ascontiguousarray(ipiv, dtype=np.int32).reshape(-1)
    batch = LU.size // (n * n)
    if LU.size != batch * n * n or B.size != batch * n * nrhs or P.size != batch * n:
        raise ValueError("LU, ipiv and B sizes do not agree")
    X = np.empty_like(B)
    rc = getattr(_load(), "oracle_getrs_" + sfx)(
        _LAYOUTS[layout], n, nrhs, batch, _ptr(LU, ct), _ptr(P, ctypes.c_int32), _ptr(B, ct),
        _ptr(X, ct), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_getrs_{sfx} returned {rc}")
    return X.reshape(np.shape(B_store))


def potrf(A_store: np.ndarray, n: int, layout: str = "row", shift: float = 0.0,
          nthreads: int = 0):
    """Cholesky factors of A + shift I.  Returns ``(L, info)``: L float
    [batch, n, n] logical row-major (lower triangular, zero above; all +0.0
    for a failed system), info int32 [batch] (0; -1 for a non-finite entry of
    A; -2 for a matrix that is not exactly symmetric; j+1 for the first
    non-positive pivot; -3 for a non-finite entry of L)."""
    sfx, ct = _sfx(A_store.dtype)
    A = np.ascontiguousarray(A_store).reshape(-1)
    batch = A.size // (n * n)
    if A.size != batch * n * n:
        raise ValueError("A size is not a multiple of n*n")
    L = np.empty((batch, n, n), dtype=A.dtype)
    info = np.empty((batch,), dtype=np.int32)
    rc = getattr(_load(), "oracle_potrf_" + sfx)(
        _LAYOUTS[layout], n, batch, float(shift), _ptr(A, ct), _ptr(L, ct),
        _ptr(info, ctypes.c_int32), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_potrf_{sfx} returned {rc}")
    return L, info


def potrs(L_store: np.ndarray, B_store: np.ndarray, n: int, nrhs: int, layout: str = "row",
          nthreads: int = 0) -> np.ndarray:
    """Solve from Cholesky factors: ``L_store`` is the storage (in
    ``layout``) of L as potrf writes it (lower triangle read; a system whose
    L(0,0) is 0, a failed factorization, gets X = +0.0).  Returns X in B's
    storage."""
    sfx, ct = _sfx(L_store.dtype)
    if np.dtype(B_store.dtype) != np.dtype(L_store.dtype):
        raise TypeError("L and B must share a dtype")
    L = np.ascontiguousarray(L_store).reshape(-1)
    B = np.ascontiguousarray(B_store).reshape(-1)
    batch = L.size // (n * n)
    if L.size != batch * n * n or B.size != batch * n * nrhs:
        raise ValueError("L and B sizes do not agree")
    X = np.empty_like(B)
    rc = getattr(_load(), "oracle_potrs_" + sfx)(
        _LAYOUTS[layout], n, nrhs, batch, _ptr(L, ct), _ptr(B, ct), _ptr(X, ct), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_potrs_{sfx} returned {rc}")
    return X.reshape(np.shape(B_store))


def posv(A_store: np.ndarray, B_store: np.ndarray, n: int, nrhs: int, layout: str = "row",
         shift: float = 0.0, nthreads: int = 0):
    """Solve (A + shift I) X = B by Cholesky.  Returns ``(X_store, info)``
    with the status of ``potrf``; a failed system gets X = +0.0."""
    sfx, ct = _sfx(A_store.dtype)
    A = np.ascontiguousarray(A_store).reshape(-1)
    B = np.ascontiguousarray(B_store).reshape(-1)
    batch = A.size // (n * n)
    if A.size != batch * n * n or B.size != batch * n * nrhs:
        raise ValueError("A and B sizes do not agree")
    X = np.empty_like(B)
    info = np.empty((batch,), dtype=np.int32)
    rc = getattr(_load(), "oracle_posv_" + sfx)(
        _LAYOUTS[layout], n, nrhs, batch, float(shift), _ptr(A, ct), _ptr(B, ct), _ptr(X, ct),
        _ptr(info, ctypes.c_int32), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_posv_{sfx} returned {rc}")
    return X.reshape(np.shape(B_store)), info


def pivot_gap(A_store: np.ndarray, n: int, layout: str = "row", nthreads: int = 0) -> np.ndarray:
    """Smallest relative pivot-candidate gap of each matrix (see ``getrf``)."""
    return getrf(A_store, n, layout, nthreads)[3]
