"""ctypes binding of libtdls.so: argument marshalling only.

Every computation happens in the library's HIP kernels; this module turns
torch tensors into the raw pointers, sizes and stream of the C interface and
allocates the outputs.  There is no fallback: without the built library, or
without a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

F32, F64 = 0, 1
ROW_MAJOR, COL_MAJOR = 0, 1
_LAYOUTS = {"row": ROW_MAJOR, "col": COL_MAJOR}

_lib = None


class TdlsError(RuntimeError):
    """A non-zero return code of the C interface."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


class Plan(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("nrhs", ctypes.c_int), ("n_kernel", ctypes.c_int),
                ("nrhs_kernel", ctypes.c_int), ("group_size", ctypes.c_int),
                ("rows_per_lane", ctypes.c_int), ("systems_per_wave", ctypes.c_int),
                ("threads_per_block", ctypes.c_int), ("systems_per_block", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class Options(ctypes.Structure):
    """tdls_options of the *_ex calls."""
    _fields_ = [("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("interleave", ctypes.c_int64)]


SCALE_MAXABS = 1

EXPORTED = ("tdls_gesv_batched", "tdls_gesv_batched_ex", "tdls_getrf_batched",
            "tdls_getrf_batched_ex", "tdls_getrs_batched", "tdls_plan_gesv", "tdls_plan_op",
            "tdls_posv_batched", "tdls_potrf_batched", "tdls_strerror", "tdls_version")
OP_GESV, OP_GETRF, OP_GETRS, OP_POTRF, OP_POSV = 0, 1, 2, 3, 4
_OPS = {"gesv": OP_GESV, "getrf": OP_GETRF, "getrs": OP_GETRS, "potrf": OP_POTRF,
        "posv": OP_POSV}


def library_path() -> str:
    return _build.library_path()


def load_library():
    """Load libtdls.so (building it first only when no build exists)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.tdls_gesv_batched.restype = ctypes.c_int
    lib.tdls_gesv_batched.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.tdls_gesv_batched_ex.restype = ctypes.c_int
    lib.tdls_gesv_batched_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int64, ctypes.POINTER(Options),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_getrf_batched_ex.restype = ctypes.c_int
    lib.tdls_getrf_batched_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.POINTER(Options),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_plan_gesv.restype = ctypes.c_int
    lib.tdls_plan_gesv.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int64, ctypes.POINTER(Plan)]
    lib.tdls_getrf_batched.restype = ctypes.c_int
    lib.tdls_getrf_batched.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_getrs_batched.restype = ctypes.c_int
    lib.tdls_getrs_batched.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_potrf_batched.restype = ctypes.c_int
    lib.tdls_potrf_batched.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_posv_batched.restype = ctypes.c_int
    lib.tdls_posv_batched.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_double, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.tdls_plan_op.restype = ctypes.c_int
    lib.tdls_plan_op.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int64, ctypes.POINTER(Plan)]
    lib.tdls_strerror.restype = ctypes.c_char_p
    lib.tdls_strerror.argtypes = [ctypes.c_int]
    lib.tdls_version.restype = ctypes.c_char_p
    lib.tdls_version.argtypes = []
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().tdls_strerror(int(code)).decode()


def version() -> str:
    return load_library().tdls_version().decode()


def tdls_gesv_batched(dtype: int, layout: int, n: int, nrhs: int, batch: int, A: int, B: int,
                      X: int, piv: int, info: int, stream: int) -> int:
    """The C call itself, raw pointers (ints) in, return code out."""
    return int(load_library().tdls_gesv_batched(int(dtype), int(layout), int(n), int(nrhs),
                                                int(batch), A, B, X, piv, info, stream))


def _opt(opt):
    return ctypes.byref(opt) if opt is not None else None


def tdls_gesv_batched_ex(dtype: int, layout: int, n: int, nrhs: int, batch: int, opt, A: int,
                         B: int, X: int, piv: int, info: int, stream: int) -> int:
    """The C call with options (an Options or None), raw pointers in."""
    return int(load_library().tdls_gesv_batched_ex(int(dtype), int(layout), int(n), int(nrhs),
                                                   int(batch), _opt(opt), A, B, X, piv, info,
                                                   stream))


def tdls_getrf_batched_ex(dtype: int, layout: int, n: int, batch: int, opt, A: int, LU: int,
                          piv: int, info: int, stream: int) -> int:
    """The C call with options (an Options or None), raw pointers in."""
    return int(load_library().tdls_getrf_batched_ex(int(dtype), int(layout), int(n), int(batch),
                                                    _opt(opt), A, LU, piv, info, stream))


def tdls_plan_gesv(dtype: int, layout: int, n: int, nrhs: int, batch: int):
    """The planner call: returns (code, Plan)."""
    p = Plan()
    rc = int(load_library().tdls_plan_gesv(int(dtype), int(layout), int(n), int(nrhs),
                                           int(batch), ctypes.byref(p)))
    return rc, p


def plan_gesv(dtype: str, layout: str, n: int, nrhs: int, batch: int) -> dict:
    rc, p = tdls_plan_gesv(F64 if dtype == "f64" else F32, _LAYOUTS[layout], n, nrhs, batch)
    if rc != 0:
        raise TdlsError(rc, "tdls_plan_gesv")
    return p.as_dict()


def tdls_getrf_batched(dtype: int, layout: int, n: int, batch: int, A: int, LU: int, piv: int,
                       info: int, stream: int) -> int:
    """The C call itself, raw pointers (ints) in, return code out."""
    return int(load_library().tdls_getrf_batched(int(dtype), int(layout), int(n), int(batch),
                                                 A, LU, piv, info, stream))


def tdls_getrs_batched(dtype: int, layout: int, n: int, nrhs: int, batch: int, LU: int, piv: int,
                       B: int, X: int, stream: int) -> int:
    """The C call itself, raw pointers (ints) in, return code out."""
    return int(load_library().tdls_getrs_batched(int(dtype), int(layout), int(n), int(nrhs),
                                                 int(batch), LU, piv, B, X, stream))


def tdls_potrf_batched(dtype: int, layout: int, n: int, batch: int, shift: float, A: int, L: int,
                       info: int, stream: int) -> int:
    """The C call itself, raw pointers (ints) in, return code out."""
    return int(load_library().tdls_potrf_batched(int(dtype), int(layout), int(n), int(batch),
                                                 float(shift), A, L, info, stream))


def tdls_posv_batched(dtype: int, layout: int, n: int, nrhs: int, batch: int, shift: float,
                      A: int, B: int, X: int, info: int, stream: int) -> int:
    """The C call itself, raw pointers (ints) in, return code out."""
    return int(load_library().tdls_posv_batched(int(dtype), int(layout), int(n), int(nrhs),
                                                int(batch), float(shift), A, B, X, info, stream))


def tdls_plan_op(op: int, dtype: int, layout: int, n: int, nrhs: int, batch: int):
    """The generic planner call: returns (code, Plan)."""
    p = Plan()
    rc = int(load_library().tdls_plan_op(int(op), int(dtype), int(layout), int(n), int(nrhs),
                                         int(batch), ctypes.byref(p)))
    return rc, p


def plan_op(op: str, dtype: str, layout: str, n: int, nrhs: int, batch: int) -> dict:
    rc, p = tdls_plan_op(_OPS[op], F64 if dtype == "f64" else F32, _LAYOUTS[layout], n, nrhs,
                         batch)
    if rc != 0:
        raise TdlsError(rc, "tdls_plan_op")
    return p.as_dict()


def _torch():
    import torch
    return torch


def gesv_batched(A, B, layout: str = "row", out=None, stream=None, scale: bool = False):
    """Solve a batch of systems held in torch CUDA tensors.

    A: [batch, n, n] storage of the matrices in ``layout`` (for "col" each
    A[s] holds the transpose of the logical matrix).  B: [batch, n, nrhs]
    ("row") or [batch, nrhs, n] ("col").  float32 or float64, contiguous,
    same device.  Returns (X, piv, info) with X shaped like B, piv int32
    [batch, n], info int32 [batch] (0; -1 non-finite input; k first zero
    pivot; -3 non-finite result).  ``out`` may pass preallocated (X, piv,
    info).  ``scale`` selects the whole-matrix max-abs scaling.  Runs on
    ``stream`` (default: the current stream) and does not synchronize.
    """
    torch = _torch()
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'row' or 'col'")
    if A.dtype not in (torch.float32, torch.float64) or B.dtype != A.dtype:
        raise TypeError("A and B must both be float32 or both float64")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be CUDA tensors on the same device")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous")
    if A.dim() != 3 or A.shape[1] != A.shape[2]:
        raise ValueError("A must be [batch, n, n]")
    batch, n = A.shape[0], A.shape[1]
    if B.dim() != 3 or B.shape[0] != batch:
        raise ValueError("B must be [batch, n, nrhs] (row) or [batch, nrhs, n] (col)")
    nrhs = B.shape[2] if layout == "row" else B.shape[1]
    if (B.shape[1] if layout == "row" else B.shape[2]) != n:
        raise ValueError("B does not match n")
    if out is None:
        X = torch.empty_like(B)
        piv = torch.empty((batch, n), dtype=torch.int32, device=A.device)
        info = torch.empty((batch,), dtype=torch.int32, device=A.device)
    else:
        X, piv, info = out
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    dt = F64 if A.dtype == torch.float64 else F32
    with torch.cuda.device(A.device):
        if scale:
            rc = tdls_gesv_batched_ex(dt, _LAYOUTS[layout], n, nrhs, batch,
                                      Options(SCALE_MAXABS, 0, 1), A.data_ptr(), B.data_ptr(),
                                      X.data_ptr(), piv.data_ptr(), info.data_ptr(),
                                      s.cuda_stream)
        else:
            rc = tdls_gesv_batched(dt, _LAYOUTS[layout], n, nrhs, batch, A.data_ptr(),
                                   B.data_ptr(), X.data_ptr(), piv.data_ptr(), info.data_ptr(),
                                   s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_gesv_batched")
    return X, piv, info


def _check_square(torch, A, name):
    if A.dtype not in (torch.float32, torch.float64):
        raise TypeError(f"{name} must be float32 or float64")
    if not A.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not A.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if A.dim() != 3 or A.shape[1] != A.shape[2]:
        raise ValueError(f"{name} must be [batch, n, n]")


def getrf_batched(A, layout: str = "row", out=None, stream=None, scale: bool = False):
    """Factor a batch of matrices held in torch CUDA tensors: P A = L U.

    A: [batch, n, n] storage in ``layout``.  Returns (LU, piv, info): LU like
    A (LAPACK's row order, unit-lower L below the diagonal, U on and above
    it, in the same layout), piv int32 [batch, n] (0-based swap sequence, -1
    for a failed system), info int32 [batch].  ``scale``: whole-matrix
    max-abs scaling, U multiplied back at the end.  Does not synchronize.
    """
    torch = _torch()
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'row' or 'col'")
    _check_square(torch, A, "A")
    batch, n = A.shape[0], A.shape[1]
    if out is None:
        LU = torch.empty_like(A)
        piv = torch.empty((batch, n), dtype=torch.int32, device=A.device)
        info = torch.empty((batch,), dtype=torch.int32, device=A.device)
    else:
        LU, piv, info = out
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    dt = F64 if A.dtype == torch.float64 else F32
    with torch.cuda.device(A.device):
        if scale:
            rc = tdls_getrf_batched_ex(dt, _LAYOUTS[layout], n, batch,
                                       Options(SCALE_MAXABS, 0, 1), A.data_ptr(), LU.data_ptr(),
                                       piv.data_ptr(), info.data_ptr(), s.cuda_stream)
        else:
            rc = tdls_getrf_batched(dt, _LAYOUTS[layout], n, batch, A.data_ptr(), LU.data_ptr(),
                                    piv.data_ptr(), info.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_getrf_batched")
    return LU, piv, info


def getrs_batched(LU, piv, B, layout: str = "row", out=None, stream=None):
    """Solve from factors of getrf_batched: X with A X = B.

    LU: [batch, n, n] and piv int32 [batch, n] as returned by getrf_batched
    (same layout); B: [batch, n, nrhs] ("row") or [batch, nrhs, n] ("col").
    Returns X shaped like B.  Does not synchronize.
    """
    torch = _torch()
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'row' or 'col'")
    _check_square(torch, LU, "LU")
    batch, n = LU.shape[0], LU.shape[1]
    if B.dtype != LU.dtype or not B.is_cuda or B.device != LU.device or not B.is_contiguous():
        raise ValueError("B must be a contiguous CUDA tensor of LU's dtype and device")
    if piv.dtype != torch.int32 or piv.device != LU.device or not piv.is_contiguous() \
            or tuple(piv.shape) != (batch, n):
        raise ValueError("piv must be a contiguous int32 [batch, n] tensor on LU's device")
    if B.dim() != 3 or B.shape[0] != batch:
        raise ValueError("B must be [batch, n, nrhs] (row) or [batch, nrhs, n] (col)")
    nrhs = B.shape[2] if layout == "row" else B.shape[1]
    if (B.shape[1] if layout == "row" else B.shape[2]) != n:
        raise ValueError("B does not match n")
    X = torch.empty_like(B) if out is None else out
    s = stream if stream is not None else torch.cuda.current_stream(LU.device)
    with torch.cuda.device(LU.device):
        rc = tdls_getrs_batched(F64 if LU.dtype == torch.float64 else F32, _LAYOUTS[layout], n,
                                nrhs, batch, LU.data_ptr(), piv.data_ptr(), B.data_ptr(),
                                X.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_getrs_batched")
    return X


def potrf_batched(A, layout: str = "row", shift: float = 0.0, out=None, stream=None):
    """Cholesky factors of a batch of symmetric matrices: A + shift I = L L^T.

    A: [batch, n, n] in ``layout`` (exactly symmetric, else info = -2).
    Returns (L, info): L like A, lower triangular with +0.0 above (all +0.0
    for a failed system); info int32 [batch] (0, j for the first leading
    minor that is not positive definite, -2).  Does not synchronize.
    """
    torch = _torch()
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'row' or 'col'")
    _check_square(torch, A, "A")
    batch, n = A.shape[0], A.shape[1]
    if out is None:
        L = torch.empty_like(A)
        info = torch.empty((batch,), dtype=torch.int32, device=A.device)
    else:
        L, info = out
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        rc = tdls_potrf_batched(F64 if A.dtype == torch.float64 else F32, _LAYOUTS[layout], n,
                                batch, shift, A.data_ptr(), L.data_ptr(), info.data_ptr(),
                                s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_potrf_batched")
    return L, info


def posv_batched(A, B, layout: str = "row", shift: float = 0.0, out=None, stream=None):
    """Solve (A + shift I) X = B by Cholesky for a batch of symmetric
    positive definite systems.  Shapes as for gesv_batched.  Returns (X,
    info) with potrf_batched's status; a failed system gets X = +0.0."""
    torch = _torch()
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'row' or 'col'")
    _check_square(torch, A, "A")
    batch, n = A.shape[0], A.shape[1]
    if B.dtype != A.dtype or not B.is_cuda or B.device != A.device or not B.is_contiguous():
        raise ValueError("B must be a contiguous CUDA tensor of A's dtype and device")
    if B.dim() != 3 or B.shape[0] != batch:
        raise ValueError("B must be [batch, n, nrhs] (row) or [batch, nrhs, n] (col)")
    nrhs = B.shape[2] if layout == "row" else B.shape[1]
    if (B.shape[1] if layout == "row" else B.shape[2]) != n:
        raise ValueError("B does not match n")
    if out is None:
        X = torch.empty_like(B)
        info = torch.empty((batch,), dtype=torch.int32, device=A.device)
    else:
        X, info = out
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        rc = tdls_posv_batched(F64 if A.dtype == torch.float64 else F32, _LAYOUTS[layout], n,
                               nrhs, batch, shift, A.data_ptr(), B.data_ptr(), X.data_ptr(),
                               info.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_posv_batched")
    return X, info
