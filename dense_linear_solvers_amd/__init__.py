"""MI355X (gfx950) batched small dense linear solver.

``gesv_batched`` solves many independent n x n systems (n <= 64, up to 8
right-hand sides, float32 or float64) by LU with partial row pivoting plus
forward and back substitution; ``getrf_batched`` writes the factors and
``getrs_batched`` solves from them; ``potrf_batched``, ``potrs_batched``
and ``posv_batched`` do the same for symmetric positive definite systems by
Cholesky.  All of it runs in hand-written HIP
kernels behind the C interface of include/tdls.h.  PyTorch only supplies device memory and
streams.
"""
from ._binding import (COL_MAJOR, EXPORTED, F32, F64, OP_GESV, OP_GETRF, OP_GETRS, OP_POSV,
                       OP_POTRF, OP_POTRS, ROW_MAJOR, SCALE_MAXABS, Options, Plan, TdlsError, gesv_batched,
                       getrf_batched, getrs_batched, library_path, load_library, plan_gesv,
                       plan_op, posv_batched, potrf_batched, potrs_batched, strerror,
                       tdls_gesv_batched,
                       tdls_gesv_batched_ex, tdls_getrf_batched, tdls_getrf_batched_ex,
                       tdls_getrs_batched, tdls_getrs_batched_ex, tdls_plan_gesv, tdls_plan_op,
                       tdls_posv_batched, tdls_posv_batched_ex, tdls_potrf_batched,
                       tdls_potrf_batched_ex, tdls_potrs_batched, tdls_potrs_batched_ex, version)

__all__ = ["gesv_batched", "getrf_batched", "getrs_batched", "potrf_batched", "potrs_batched",
           "posv_batched", "plan_gesv", "plan_op", "strerror", "version", "library_path",
           "load_library", "tdls_gesv_batched", "tdls_gesv_batched_ex", "tdls_getrf_batched",
           "tdls_getrf_batched_ex", "tdls_getrs_batched", "tdls_getrs_batched_ex",
           "tdls_potrf_batched", "tdls_potrf_batched_ex", "tdls_potrs_batched",
           "tdls_potrs_batched_ex", "tdls_posv_batched", "tdls_posv_batched_ex", "tdls_plan_gesv",
           "tdls_plan_op", "TdlsError", "Plan", "Options", "EXPORTED", "F32", "F64", "ROW_MAJOR",
           "COL_MAJOR", "SCALE_MAXABS", "OP_GESV", "OP_GETRF", "OP_GETRS", "OP_POTRF", "OP_POSV",
           "OP_POTRS"]
