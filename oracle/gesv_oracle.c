/*
 * CPU oracle for batched gesv: LU factorization with partial row pivoting,
 * then forward and back substitution, one system at a time.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * GPU path is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no source, header
 * or constant with the GPU library (the enum values below are restated from
 * the meaning of the arguments, not included from the library's header).
 *
 * What it computes, and where that is stated:
 *  - The elimination is the right-looking LU with partial pivoting described
 *    on the cooperative LU solver page ("solver_static.hpp File Reference",
 *    Detailed Description): P A = L U, the forward substitution L y = P b
 *    folded into the factorization, then U x = y.  The layout flag only
 *    changes addressing: rows of A are pivoted in both layouts (the row-major
 *    case of that page pivots columns of A; the ruSOLVER page fixes partial
 *    row pivoting on row-major [batch, n, n] input, which is the reading
 *    taken here).
 *  - Pivot ties go to the lowest current row position, and multipliers are
 *    exact quotients, not products with a reciprocal ("ruSOLVER：小矩阵 kernel
 *    优化（实验性）", section on the unchanged numerical and failure contract:
 *    lowest-row-number tie rule, no reciprocal approximation).
 *  - Status: 0 on success, k >= 1 for the first failing pivot, here a pivot
 *    that is exactly zero (same section; the cuSolverDx POTRF page uses the
 *    same 1-based first-failure index).  A failed system has an all-zero
 *    solution and every pivot entry -1 (same section).
 *  - piv[k] is the 0-based LAPACK swap sequence: the position exchanged with
 *    k at step k.
 *
 * The same file holds the Cholesky factorization and solve of symmetric
 * positive definite systems (potrf, posv) under the ruSOLVER contract for
 * that path: exact symmetry check (status -2), explicit diagonal shift,
 * inner products in increasing k, status j+1 for the first non-positive
 * pivot, failed systems zeroed.
 *
 * The non-finite statuses of the same contract hold everywhere: -1 for a
 * non-finite input entry, -3 for a non-finite computed value (after the
 * positive status of a failed pivot in precedence).  Its whole-matrix
 * max-abs scaling of the LU, with the scale of U restored, is an option of
 * gesv and getrf (`scale`).
 *
 * Built with gcc -O2 -ffp-contract=off so that no multiply-add is fused
 * except the explicit fma()/fmaf() calls, which match the GPU's fused
 * multiply-adds one for one.  OpenMP runs the independent systems in
 * parallel; each system is computed serially.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_ROW_MAJOR 0
#define ORACLE_COL_MAJOR 1
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static int oracle_check_args(int layout, int n, int nrhs, int64_t batch)
{
    if (layout != ORACLE_ROW_MAJOR && layout != ORACLE_COL_MAJOR)
        return ORACLE_EINVAL;
    if (n < 1 || nrhs < 1 || batch < 0)
        return ORACLE_EINVAL;
    return 0;
}

#define REAL double
#define SFX(x) x##_f64
#define FMA fma
#define FABS fabs
#define SQRT sqrt
#include "gesv_oracle_impl.h"
#undef REAL
#undef SFX
#undef FMA
#undef FABS
#undef SQRT

#define REAL float
#define SFX(x) x##_f32
#define FMA fmaf
#define FABS fabsf
#define SQRT sqrtf
#include "gesv_oracle_impl.h"
#undef REAL
#undef SFX
#undef FMA
#undef FABS
#undef SQRT

int oracle_max_threads(void) { return omp_get_max_threads(); }
