"""MI355X (gfx950) batched small dense linear solver.

``gesv_batched`` solves many independent n x n systems (n <= 64, up to 8
right-hand sides, float32 or float64) by LU with partial row pivoting plus
forward and back substitution, in hand-written HIP kernels behind the C
interface of include/tdls.h.  PyTorch only supplies device memory and
streams.
"""
from ._binding import (COL_MAJOR, EXPORTED, F32, F64, ROW_MAJOR, Plan, TdlsError, gesv_batched,
                       library_path, load_library, plan_gesv, strerror, tdls_gesv_batched,
                       tdls_plan_gesv, version)

__all__ = ["gesv_batched", "plan_gesv", "strerror", "version", "library_path", "load_library",
           "tdls_gesv_batched", "tdls_plan_gesv", "TdlsError", "Plan", "EXPORTED", "F32", "F64",
           "ROW_MAJOR", "COL_MAJOR"]
