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
            "tdls_getrf_batched_ex", "tdls_getrs_batched", "tdls_getrs_batched_ex",
            "tdls_plan_gesv", "tdls_plan_op", "tdls_posv_batched", "tdls_posv_batched_ex",
            "tdls_potrf_batched", "tdls_potrf_batched_ex", "tdls_potrs_batched",
            "tdls_potrs_batched_ex", "tdls_strerror", "tdls_version")
OP_GESV, OP_GETRF, OP_GETRS, OP_POTRF, OP_POSV, OP_POTRS = 0, 1, 2, 3, 4, 5
_OPS = {"gesv": OP_GESV, "getrf": OP_GETRF, "getrs": OP_GETRS, "potrf": OP_POTRF,
        "posv": OP_POSV, "potrs": OP_POTRS}


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
    lib.tdls_getrs_batched_ex.restype = ctypes.c_int
    lib.tdls_getrs_batched_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.POINTER(Options),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_potrf_batched_ex.restype = ctypes.c_int
    lib.tdls_potrf_batched_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_double,
                                          ctypes.POINTER(Options), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_posv_batched_ex.restype = ctypes.c_int
    lib.tdls_posv_batched_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_double,
                                         ctypes.POINTER(Options), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.tdls_potrs_batched.restype = ctypes.c_int
    lib.tdls_potrs_batched.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.tdls_potrs_batched_ex.restype = ctypes.c_int
    lib.tdls_potrs_batched_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.POINTER(Options),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
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


def tdls_getrs_batched_ex(dtype: int, layout: int, n: int, nrhs: int, batch: int, opt, LU: int,
                          piv: int, B: int, X: int, stream: int) -> int:
    """The C call with options (an Options or None), raw pointers in."""
    return int(load_library().tdls_getrs_batched_ex(int(dtype), int(layout), int(n), int(nrhs),
                                                    int(batch), _opt(opt), LU, piv, B, X,
                                                    stream))


def tdls_potrf_batched_ex(dtype: int, layout: int, n: int, batch: int, shift: float, opt, A: int,
                          L: int, info: int, stream: int) -> int:
    """The C call with options (an Options or None), raw pointers in."""
    return int(load_library().tdls_potrf_batched_ex(int(dtype), int(layout), int(n), int(batch),
                                                    float(shift), _opt(opt), A, L, info, stream))


def tdls_posv_batched_ex(dtype: int, layout: int, n: int, nrhs: int, batch: int, shift: float,
                         opt, A: int, B: int, X: int, info: int, stream: int) -> int:
    """The C call with options (an Options or None), raw pointers in."""
    return int(load_library().tdls_posv_batched_ex(int(dtype), int(layout), int(n), int(nrhs),
                                                   int(batch), float(shift), _opt(opt), A, B, X,
                                                   info, stream))


def tdls_potrs_batched(dtype: int, layout: int, n: int, nrhs: int, batch: int, L: int, B: int,
                       X: int, stream: int) -> int:
    """The C call itself, raw pointers (ints) in, return code out."""
    return int(load_library().tdls_potrs_batched(int(dtype), int(layout), int(n), int(nrhs),
                                                 int(batch), L, B, X, stream))


def tdls_potrs_batched_ex(dtype: int, layout: int, n: int, nrhs: int, batch: int, opt, L: int,
                          B: int, X: int, stream: int) -> int:
    """The C call with options (an Options or None), raw pointers in."""
    return int(load_library().tdls_potrs_batched_ex(int(dtype), int(layout), int(n), int(nrhs),
                                                    int(batch), _opt(opt), L, B, X, stream))


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


def _dtype_code(torch, A):
    return F64 if A.dtype == torch.float64 else F32


def _check_pair(torch, A, B, nameA="A", nameB="B"):
    if A.dtype not in (torch.float32, torch.float64) or B.dtype != A.dtype:
        raise TypeError(f"{nameA} and {nameB} must both be float32 or both float64")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError(f"{nameA} and {nameB} must be CUDA tensors on the same device")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError(f"{nameA} and {nameB} must be contiguous")


def _check_square(torch, A, name):
    if A.dtype not in (torch.float32, torch.float64):
        raise TypeError(f"{name} must be float32 or float64")
    if not A.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not A.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if A.dim() != 3 or A.shape[1] != A.shape[2]:
        raise ValueError(f"{name} must be [batch, n, n]")


def _check_out(torch, t, name, dtype, device, shape):
    """An ``out`` tensor must be exactly what the call would allocate: the
    library sees raw pointers only, so a wrong size, type or device would be
    written past or to the wrong memory.  Raises before any library call."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"out {name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"out {name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"out {name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"out {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"out {name} must be contiguous")


def _unpack_out(out, names):
    if len(names) == 1:
        return (out,)
    if not isinstance(out, (tuple, list)) or len(out) != len(names):
        raise TypeError(f"out must be a tuple ({', '.join(names)})")
    return tuple(out)


def _interleaved_dims(A, B, layout: str, interleave: int, batch):
    """Problem sizes of interleaved operands: A [blocks, n, n, W] and B
    [blocks, n, nrhs, W] ("row") or [blocks, nrhs, n, W] ("col"), system s
    in slice [s // W, ..., s % W]; ``batch`` defaults to blocks * W."""
    W = int(interleave)
    if A.dim() != 4 or A.shape[1] != A.shape[2] or A.shape[3] != W:
        raise ValueError("interleaved A must be [blocks, n, n, W]")
    blocks, n = A.shape[0], A.shape[1]
    b = blocks * W if batch is None else int(batch)
    if not ((blocks - 1) * W < b <= blocks * W or (b == 0 and blocks == 0)):
        raise ValueError("batch does not match the interleaved blocks")
    nrhs = None
    if B is not None:
        if B.dim() != 4 or B.shape[0] != blocks or B.shape[3] != W:
            raise ValueError("interleaved B must be [blocks, n, nrhs, W] (row) or "
                             "[blocks, nrhs, n, W] (col)")
        nrhs = B.shape[2] if layout == "row" else B.shape[1]
        if (B.shape[1] if layout == "row" else B.shape[2]) != n:
            raise ValueError("B does not match n")
    return b, n, nrhs


def _plain_dims(A, B, layout):
    if A.dim() != 3 or A.shape[1] != A.shape[2]:
        raise ValueError("A must be [batch, n, n]")
    batch, n = A.shape[0], A.shape[1]
    nrhs = None
    if B is not None:
        if B.dim() != 3 or B.shape[0] != batch:
            raise ValueError("B must be [batch, n, nrhs] (row) or [batch, nrhs, n] (col)")
        nrhs = B.shape[2] if layout == "row" else B.shape[1]
        if (B.shape[1] if layout == "row" else B.shape[2]) != n:
            raise ValueError("B does not match n")
    return batch, n, nrhs


def _dims(A, B, layout, interleave, batch):
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'row' or 'col'")
    if interleave > 1:
        return _interleaved_dims(A, B, layout, interleave, batch)
    if batch is not None and batch != A.shape[0]:
        raise ValueError("batch is given by A's first dimension")
    return _plain_dims(A, B, layout)


def _piv_shape(A, n, interleave):
    return (A.shape[0], n, interleave) if interleave > 1 else (A.shape[0], n)


def _options(flags, interleave):
    return Options(flags, 0, max(1, int(interleave)))


# Interleaved batches (``interleave`` W > 1): the operands are 4-D, A
# [blocks, n, n, W] (its [b, :, :, w] slice is system b*W + w in ``layout``),
# B and X [blocks, n, nrhs, W] ("row") or [blocks, nrhs, n, W] ("col"), piv
# [blocks, n, W]; info stays [batch].  ``batch`` may end inside the last
# block.  W = 1 (default): the 3-D operands of the plain calls.


def gesv_batched(A, B, layout: str = "row", out=None, stream=None, scale: bool = False,
                 interleave: int = 1, batch=None):
    """Solve a batch of systems held in torch CUDA tensors.

    A: [batch, n, n] storage of the matrices in ``layout`` (for "col" each
    A[s] holds the transpose of the logical matrix).  B: [batch, n, nrhs]
    ("row") or [batch, nrhs, n] ("col").  float32 or float64, contiguous,
    same device.  Returns (X, piv, info) with X shaped like B, piv int32
    [batch, n], info int32 [batch] (0; -1 non-finite input; k first zero
    pivot; -3 non-finite result).  ``out`` may pass preallocated (X, piv,
    info).  ``scale`` selects the whole-matrix max-abs scaling;
    ``interleave`` an interleaved batch (see above).  Runs on ``stream``
    (default: the current stream) and does not synchronize.
    """
    torch = _torch()
    _check_pair(torch, A, B)
    nb, n, nrhs = _dims(A, B, layout, interleave, batch)
    if out is None:
        X = torch.empty_like(B)
        piv = torch.empty(_piv_shape(A, n, interleave), dtype=torch.int32, device=A.device)
        info = torch.empty((nb,), dtype=torch.int32, device=A.device)
    else:
        X, piv, info = _unpack_out(out, ("X", "piv", "info"))
        _check_out(torch, X, "X", B.dtype, B.device, B.shape)
        _check_out(torch, piv, "piv", torch.int32, A.device, _piv_shape(A, n, interleave))
        _check_out(torch, info, "info", torch.int32, A.device, (nb,))
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    dt = _dtype_code(torch, A)
    with torch.cuda.device(A.device):
        if scale or interleave > 1:
            rc = tdls_gesv_batched_ex(dt, _LAYOUTS[layout], n, nrhs, nb,
                                      _options(SCALE_MAXABS if scale else 0, interleave),
                                      A.data_ptr(), B.data_ptr(), X.data_ptr(), piv.data_ptr(),
                                      info.data_ptr(), s.cuda_stream)
        else:
            rc = tdls_gesv_batched(dt, _LAYOUTS[layout], n, nrhs, nb, A.data_ptr(),
                                   B.data_ptr(), X.data_ptr(), piv.data_ptr(), info.data_ptr(),
                                   s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_gesv_batched")
    return X, piv, info


def getrf_batched(A, layout: str = "row", out=None, stream=None, scale: bool = False,
                  interleave: int = 1, batch=None):
    """Factor a batch of matrices held in torch CUDA tensors: P A = L U.

    A: [batch, n, n] storage in ``layout``.  Returns (LU, piv, info): LU like
    A (LAPACK's row order, unit-lower L below the diagonal, U on and above
    it, in the same layout), piv int32 [batch, n] (0-based swap sequence, -1
    for a failed system), info int32 [batch].  ``scale``: whole-matrix
    max-abs scaling, U multiplied back at the end.  ``interleave``: an
    interleaved batch.  Does not synchronize.
    """
    torch = _torch()
    if A.dtype not in (torch.float32, torch.float64) or not A.is_cuda or not A.is_contiguous():
        raise ValueError("A must be a contiguous float32 or float64 CUDA tensor")
    nb, n, _ = _dims(A, None, layout, interleave, batch)
    if out is None:
        LU = torch.empty_like(A)
        piv = torch.empty(_piv_shape(A, n, interleave), dtype=torch.int32, device=A.device)
        info = torch.empty((nb,), dtype=torch.int32, device=A.device)
    else:
        LU, piv, info = _unpack_out(out, ("LU", "piv", "info"))
        _check_out(torch, LU, "LU", A.dtype, A.device, A.shape)
        _check_out(torch, piv, "piv", torch.int32, A.device, _piv_shape(A, n, interleave))
        _check_out(torch, info, "info", torch.int32, A.device, (nb,))
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    dt = _dtype_code(torch, A)
    with torch.cuda.device(A.device):
        if scale or interleave > 1:
            rc = tdls_getrf_batched_ex(dt, _LAYOUTS[layout], n, nb,
                                       _options(SCALE_MAXABS if scale else 0, interleave),
                                       A.data_ptr(), LU.data_ptr(), piv.data_ptr(),
                                       info.data_ptr(), s.cuda_stream)
        else:
            rc = tdls_getrf_batched(dt, _LAYOUTS[layout], n, nb, A.data_ptr(), LU.data_ptr(),
                                    piv.data_ptr(), info.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_getrf_batched")
    return LU, piv, info


def getrs_batched(LU, piv, B, layout: str = "row", out=None, stream=None, interleave: int = 1,
                  batch=None):
    """Solve from factors of getrf_batched: X with A X = B.

    LU: [batch, n, n] and piv int32 [batch, n] as returned by getrf_batched
    (same layout and interleave); B: [batch, n, nrhs] ("row") or [batch,
    nrhs, n] ("col").  Returns X shaped like B.  Does not synchronize.
    """
    torch = _torch()
    _check_pair(torch, LU, B, "LU", "B")
    nb, n, nrhs = _dims(LU, B, layout, interleave, batch)
    if piv.dtype != torch.int32 or piv.device != LU.device or not piv.is_contiguous() \
            or tuple(piv.shape) != _piv_shape(LU, n, interleave):
        raise ValueError("piv must be a contiguous int32 tensor on LU's device, shaped as "
                         "getrf_batched returns it")
    X = torch.empty_like(B) if out is None else out
    if out is not None:
        _check_out(torch, X, "X", B.dtype, B.device, B.shape)
    s = stream if stream is not None else torch.cuda.current_stream(LU.device)
    dt = _dtype_code(torch, LU)
    with torch.cuda.device(LU.device):
        if interleave > 1:
            rc = tdls_getrs_batched_ex(dt, _LAYOUTS[layout], n, nrhs, nb, _options(0, interleave),
                                       LU.data_ptr(), piv.data_ptr(), B.data_ptr(), X.data_ptr(),
                                       s.cuda_stream)
        else:
            rc = tdls_getrs_batched(dt, _LAYOUTS[layout], n, nrhs, nb, LU.data_ptr(),
                                    piv.data_ptr(), B.data_ptr(), X.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_getrs_batched")
    return X


def potrf_batched(A, layout: str = "row", shift: float = 0.0, out=None, stream=None,
                  interleave: int = 1, batch=None):
    """Cholesky factors of a batch of symmetric matrices: A + shift I = L L^T.

    A: [batch, n, n] in ``layout`` (exactly symmetric, else info = -2).
    Returns (L, info): L like A, lower triangular with +0.0 above (all +0.0
    for a failed system); info int32 [batch] (0; -1 non-finite input; -2;
    j for the first leading minor that is not positive definite; -3
    non-finite factor).  ``interleave``: an interleaved batch.  Does not
    synchronize.
    """
    torch = _torch()
    if A.dtype not in (torch.float32, torch.float64) or not A.is_cuda or not A.is_contiguous():
        raise ValueError("A must be a contiguous float32 or float64 CUDA tensor")
    nb, n, _ = _dims(A, None, layout, interleave, batch)
    if out is None:
        L = torch.empty_like(A)
        info = torch.empty((nb,), dtype=torch.int32, device=A.device)
    else:
        L, info = _unpack_out(out, ("L", "info"))
        _check_out(torch, L, "L", A.dtype, A.device, A.shape)
        _check_out(torch, info, "info", torch.int32, A.device, (nb,))
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    dt = _dtype_code(torch, A)
    with torch.cuda.device(A.device):
        if interleave > 1:
            rc = tdls_potrf_batched_ex(dt, _LAYOUTS[layout], n, nb, shift,
                                       _options(0, interleave), A.data_ptr(), L.data_ptr(),
                                       info.data_ptr(), s.cuda_stream)
        else:
            rc = tdls_potrf_batched(dt, _LAYOUTS[layout], n, nb, shift, A.data_ptr(),
                                    L.data_ptr(), info.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_potrf_batched")
    return L, info


def potrs_batched(L, B, layout: str = "row", out=None, stream=None, interleave: int = 1,
                  batch=None):
    """Solve from Cholesky factors of potrf_batched: X with L L^T X = B.

    L: as returned by potrf_batched (same layout and interleave; only the
    lower triangle is read; a failed factorization, all +0.0, gives X =
    +0.0); B: [batch, n, nrhs] ("row") or [batch, nrhs, n] ("col").  Returns
    X shaped like B.  Does not synchronize."""
    torch = _torch()
    _check_pair(torch, L, B, "L", "B")
    nb, n, nrhs = _dims(L, B, layout, interleave, batch)
    X = torch.empty_like(B) if out is None else out
    if out is not None:
        _check_out(torch, X, "X", B.dtype, B.device, B.shape)
    s = stream if stream is not None else torch.cuda.current_stream(L.device)
    dt = _dtype_code(torch, L)
    with torch.cuda.device(L.device):
        if interleave > 1:
            rc = tdls_potrs_batched_ex(dt, _LAYOUTS[layout], n, nrhs, nb, _options(0, interleave),
                                       L.data_ptr(), B.data_ptr(), X.data_ptr(), s.cuda_stream)
        else:
            rc = tdls_potrs_batched(dt, _LAYOUTS[layout], n, nrhs, nb, L.data_ptr(), B.data_ptr(),
                                    X.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_potrs_batched")
    return X


def posv_batched(A, B, layout: str = "row", shift: float = 0.0, out=None, stream=None,
                 interleave: int = 1, batch=None):
    """Solve (A + shift I) X = B by Cholesky for a batch of symmetric
    positive definite systems.  Shapes as for gesv_batched.  Returns (X,
    info) with potrf_batched's status (-1 also for a non-finite entry of B);
    a failed system gets X = +0.0."""
    torch = _torch()
    _check_pair(torch, A, B)
    nb, n, nrhs = _dims(A, B, layout, interleave, batch)
    if out is None:
        X = torch.empty_like(B)
        info = torch.empty((nb,), dtype=torch.int32, device=A.device)
    else:
        X, info = _unpack_out(out, ("X", "info"))
        _check_out(torch, X, "X", B.dtype, B.device, B.shape)
        _check_out(torch, info, "info", torch.int32, A.device, (nb,))
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    dt = _dtype_code(torch, A)
    with torch.cuda.device(A.device):
        if interleave > 1:
            rc = tdls_posv_batched_ex(dt, _LAYOUTS[layout], n, nrhs, nb, shift,
                                      _options(0, interleave), A.data_ptr(), B.data_ptr(),
                                      X.data_ptr(), info.data_ptr(), s.cuda_stream)
        else:
            rc = tdls_posv_batched(dt, _LAYOUTS[layout], n, nrhs, nb, shift, A.data_ptr(),
                                   B.data_ptr(), X.data_ptr(), info.data_ptr(), s.cuda_stream)
    if rc != 0:
        raise TdlsError(rc, "tdls_posv_batched")
    return X, info
