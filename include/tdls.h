/*
 * tdls.h -- C interface of the MI355X (gfx950) batched small-system solver.
 *
 * One call solves `batch` independent dense systems A_s X_s = B_s, each n x n
 * with 1..8 right-hand sides, by LU factorization with partial row pivoting
 * followed by forward and back substitution (LAPACK's gesv, one system per
 * group of lanes of a GPU wavefront).
 *
 * Where the operation is defined (page title, section):
 *   - "solver_static.hpp File Reference" (TDLS CooperativeLUpp solver),
 *     Detailed Description: right-looking LU with partial pivoting held in
 *     the registers of a group of threads, one system per group, with the
 *     forward substitution folded into the factorization and the back
 *     substitution U x = y; the layout flag of that page selects row- or
 *     column-major storage of A.
 *   - "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
 *     numerical and failure contract, and section on support and
 *     trade-offs: [batch, n, n] / [batch, n, nrhs] inputs, partial ROW
 *     pivoting with the lowest row number winning ties, no reciprocal
 *     approximation, status 0 / first failed pivot, a failed system gets
 *     zeroed results and pivots -1, inputs read-only with separate output
 *     buffers, host validation before any launch, no kernel for an empty
 *     batch and exactly one kernel otherwise, errors instead of silent
 *     fallbacks.
 *
 * Reading taken for the row-major layout: the rows of A are pivoted in both
 * layouts (P A = L U); the layout flag only changes how elements are
 * addressed.
 */
#ifndef TDLS_H
#define TDLS_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of A, B and X. */
/* In C++ the enumerations below take int as their underlying type, so any
 * int passed through the C interface is a value of the type (the calls
 * validate it and reject others with -i); without a fixed type an
 * out-of-range value would be undefined behaviour in C++.  C enumerations
 * are int-compatible already. */
#ifdef __cplusplus
#define TDLS_ENUM_BASE : int
#else
#define TDLS_ENUM_BASE
#endif

typedef enum tdls_dtype TDLS_ENUM_BASE {
  TDLS_F32 = 0, /* IEEE binary32, every operation in binary32 */
  TDLS_F64 = 1  /* IEEE binary64, every operation in binary64 */
} tdls_dtype;

/* Storage order of each system's A, B and X (the same flag for all three). */
typedef enum tdls_layout TDLS_ENUM_BASE {
  TDLS_ROW_MAJOR = 0, /* A(r,c) at r*n + c;  B(r,j), X(r,j) at r*nrhs + j */
  TDLS_COL_MAJOR = 1  /* A(r,c) at c*n + r;  B(r,j), X(r,j) at j*n + r    */
} tdls_layout;

/* Operations, for tdls_plan_op. */
typedef enum tdls_op TDLS_ENUM_BASE {
  TDLS_OP_GESV = 0,  /* factor and solve in one call (tdls_gesv_batched) */
  TDLS_OP_GETRF = 1, /* factor only (tdls_getrf_batched) */
  TDLS_OP_GETRS = 2, /* solve from factors (tdls_getrs_batched) */
  TDLS_OP_POTRF = 3, /* Cholesky factor (tdls_potrf_batched) */
  TDLS_OP_POSV = 4,  /* Cholesky factor and solve (tdls_posv_batched) */
  TDLS_OP_POTRS = 5  /* solve from Cholesky factors (tdls_potrs_batched) */
} tdls_op;

/* Return codes of the calls (not the per-system status, see `info`). */
#define TDLS_SUCCESS 0
/* -i: the i-th argument of the call is invalid (LAPACK style, 1-based). */
#define TDLS_ERR_LAUNCH (-100)      /* the HIP launch failed (see tdls_strerror) */
#define TDLS_ERR_DEVICE (-101)      /* the current device is not gfx950 */
#define TDLS_ERR_HIP (-102)         /* a HIP query failed */
#define TDLS_ERR_NO_KERNEL (-103)   /* no kernel built for the planned shape */

/* What tdls_gesv_batched would launch for a given problem (host only). */
typedef struct tdls_plan {
  int n, nrhs;               /* the problem */
  int n_kernel;              /* compile-time size the kernel is built for (>= n) */
  int nrhs_kernel;           /* compile-time right-hand sides (>= nrhs) */
  int group_size;            /* T: lanes cooperating on one system */
  int rows_per_lane;         /* R = ceil(n_kernel / T) */
  int systems_per_wave;      /* 64 / T */
  int threads_per_block;
  int64_t systems_per_block;
  int64_t grid;              /* blocks launched (0 for an empty batch) */
  int lds_bytes;             /* LDS per block */
} tdls_plan;

/*
 * Solve A_s X_s = B_s for s = 0 .. batch-1 on `stream`.
 *
 * Arguments (the number in brackets is the error code returned when the
 * argument is rejected, as -i):
 *   [1] dtype   TDLS_F32 or TDLS_F64.
 *   [2] layout  TDLS_ROW_MAJOR or TDLS_COL_MAJOR; applies to A, B and X.
 *   [3] n       1 <= n <= 64.
 *   [4] nrhs    1 <= nrhs <= 8.
 *   [5] batch   >= 0.  0 launches nothing and returns TDLS_SUCCESS.
 *   [6] A       device pointer, batch * n * n elements, system s at s*n*n;
 *               read only.  Aligned to the element size.
 *   [7] B       device pointer, batch * n * nrhs elements, system s at
 *               s*n*nrhs; read only.  Aligned to the element size.
 *   [8] X       device pointer, batch * n * nrhs elements, layout of B;
 *               written.  Must not overlap A, B, piv or info.
 *   [9] piv     device pointer, int32 [batch][n]; written.  piv[s][k] is the
 *               0-based row exchanged with row k at step k (LAPACK's swap
 *               sequence), or -1 everywhere for a failed system.
 *  [10] info    device pointer, int32 [batch]; written.  The status of
 *               the ruSOLVER contract, in this order of precedence:
 *                 -1  an entry of A or B is NaN or infinite;
 *                 k   (k >= 1) the pivot of step k (1-based) is exactly
 *                     zero, the first such step;
 *                 -3  a computed value is NaN or infinite (an entry of L,
 *                     U, L^-1 P b or x, e.g. after an overflow);
 *                 0   success.
 *               A failed system (info != 0) gets X = +0.0 and piv = -1 in
 *               every entry.  A NaN arising in a pivot search ranks above
 *               every number, so the zero-pivot status stays well defined.
 *       stream  HIP stream (0 = the null stream).
 *
 * Every output entry of every system is written, so outputs need no
 * clearing.  Ties between equal pivot magnitudes go to the lowest current
 * row position.  Multipliers and solution entries are correctly rounded
 * IEEE quotients.
 *
 * Ownership and behaviour: all buffers belong to the caller; the library
 * allocates and frees nothing, keeps no per-call state and never
 * synchronizes.  With batch > 0 exactly one kernel is enqueued on `stream`
 * and the call returns at once; results are valid once the stream has
 * reached that point.  Arguments are validated before anything is
 * enqueued; on error nothing is launched.  Results do not depend on the
 * group size chosen by the planner.
 *
 * Returns TDLS_SUCCESS, -i for an invalid i-th argument, or one of the
 * TDLS_ERR_* codes.
 */
int tdls_gesv_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                      const void* A, const void* B, void* X, int32_t* piv, int32_t* info,
                      hipStream_t stream);

/*
 * Fill *out with the launch tdls_gesv_batched would make for this problem
 * (host only: touches no device).  Validates the same scalar arguments
 * (codes -1 .. -5); returns -6 when out is NULL.
 *
 * The launch plan is a host-side object that can be checked without a GPU,
 * as the ruSOLVER page's section on building and verifying runs its
 * launch-plan tests on the host before any device suite ("ruSOLVER：小矩阵
 * kernel 优化（实验性）", 编译和验证).  The plan holds the group size T
 * (lanes per system), rows per lane, systems per wave and per block, the
 * grid and the LDS bytes of the one kernel the solve enqueues; `out` is
 * caller-owned host memory, written only on success.
 *
 * The environment variable TDLS_GROUP_SIZE, when set to a group size built
 * for the shape, overrides the planner's choice (used by the tests that
 * check results do not depend on it); an unbuilt value yields
 * TDLS_ERR_NO_KERNEL from both calls.
 */
int tdls_plan_gesv(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                   tdls_plan* out);

/*
 * Factor A_s = P_s L_s U_s for s = 0 .. batch-1 on `stream` (LAPACK's
 * getrf, the factorization half of tdls_gesv_batched).
 *
 * The elimination, pivot rule, tie rule, quotients and status are exactly
 * those of tdls_gesv_batched ("solver_static.hpp File Reference", Detailed
 * Description; "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the
 * unchanged numerical and failure contract).  The factors are written in the
 * format of the TDLS page's section Factored format under physical
 * interchanges, which is LAPACK's: row k of LU (in the layout of A) holds
 * the multipliers of L before column k (unit diagonal implied) and the row
 * of U from column k on, the pivot itself on the diagonal.
 *
 * Arguments (-i on rejection):
 *   [1] dtype, [2] layout, [3] n (1..64): as for tdls_gesv_batched.
 *   [4] batch   >= 0; 0 launches nothing.
 *   [5] A       device, batch * n * n elements; read only.
 *   [6] LU      device, batch * n * n elements, layout of A; written; must
 *               not overlap A.
 *   [7] piv     device, int32 [batch][n]; written: the 0-based swap
 *               sequence (piv[s][k] >= k), or -1 everywhere for a failed
 *               system.
 *   [8] info    device, int32 [batch]; written: as for tdls_gesv_batched,
 *               with -1 for a non-finite entry of A and -3 for a non-finite
 *               entry of L or U.  A failed system gets LU = +0.0 and piv =
 *               -1 in every entry (its factors are not usable, per the
 *               ruSOLVER contract).
 *       stream  HIP stream.
 * Ownership, stream semantics and errors as for tdls_gesv_batched.
 */
int tdls_getrf_batched(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch,
                       const void* A, void* LU, int32_t* piv, int32_t* info,
                       hipStream_t stream);

/*
 * Solve A_s X_s = B_s from factors written by tdls_getrf_batched (LAPACK's
 * getrs): the rows of B are taken in the pivoted order given by the swap
 * sequence, then L y = P b (unit lower) and U x = y, the solution entry
 * x_k = y_k / U(k,k) by IEEE division ("solver_static.hpp File Reference",
 * sections Detailed Description and Factored format).  With the same
 * layout, tdls_getrs_batched after tdls_getrf_batched yields the same bits
 * as tdls_gesv_batched.
 *
 * Arguments (-i on rejection):
 *   [1] dtype, [2] layout, [3] n (1..64), [4] nrhs (1..8), [5] batch: as for
 *               tdls_gesv_batched.
 *   [6] LU      device, batch * n * n elements; read only.
 *   [7] piv     device, int32 [batch][n]; read only.  A system whose first
 *               entry is negative (a failed factorization) gets X = +0.0.
 *               Other entries outside 0..n-1 are clamped into the matrix
 *               when the right-hand sides are gathered (no access outside
 *               the system); the result is then unspecified.
 *   [8] B       device, batch * n * nrhs elements; read only.
 *   [9] X       device, like B; written; must not overlap LU, piv or B.
 *       stream  HIP stream.
 * A zero on the diagonal of U gives non-finite entries (no status here).
 * Ownership, stream semantics and errors as for tdls_gesv_batched.
 */
int tdls_getrs_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                       const void* LU, const int32_t* piv, const void* B, void* X,
                       hipStream_t stream);

/*
 * Cholesky factorization A_s + shift I = L_s L_s^T of symmetric positive
 * definite matrices, s = 0 .. batch-1 (LAPACK's potrf, lower).
 *
 * Contract ("ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
 * numerical and failure contract; "cuSolverDx potrf" function page):
 *   - A must be exactly symmetric in the working precision (A(i,j) ==
 *     A(j,i) for every pair), else info = -2;
 *   - the shift is explicit: the diagonal is A(j,j) + shift, rounded once,
 *     and nothing else is added;
 *   - inner products accumulate in increasing k, one fused multiply-add per
 *     term; L(j,j) is the IEEE square root, L(i,j) an IEEE quotient;
 *   - info, in this order of precedence: -1 for a NaN or infinite entry
 *     of A; -2 as above; j >= 1 for the smallest leading minor that is not
 *     positive definite (the first step whose diagonal is not > 0); -3 for
 *     a NaN or infinite entry of L (e.g. an overflowing shift); else 0;
 *   - a failed system (info != 0) gets L = +0.0 everywhere.
 *
 * Arguments (-i on rejection):
 *   [1] dtype, [2] layout, [3] n (1..64): as for tdls_gesv_batched.
 *   [4] batch   >= 0; 0 launches nothing.
 *   [5] shift   finite diagonal shift (0 for none), rounded to dtype.
 *   [6] A       device, batch * n * n elements; read only.
 *   [7] L       device, batch * n * n elements, layout of A; written: L on
 *               and below the diagonal, +0.0 above; must not overlap A.
 *   [8] info    device, int32 [batch]; written.
 *       stream  HIP stream.
 * Ownership, stream semantics and errors as for tdls_gesv_batched.
 */
int tdls_potrf_batched(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch, double shift,
                       const void* A, void* L, int32_t* info, hipStream_t stream);

/*
 * Solve (L_s L_s^T) X_s = B_s from factors written by tdls_potrf_batched
 * (LAPACK's potrs, lower): L y = b, each y_j = y_j / L(j,j) by IEEE division
 * and removed from the rows below, then L^T x = y, each x_j = y_j / L(j,j)
 * removed from the rows above, every step a fused multiply-add, in the order
 * of tdls_posv_batched, so potrf then potrs gives posv's bits
 * ("ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged numerical
 * and failure contract: a failed system's factors are all zero, so a system
 * whose L(0,0) is 0 gets X = +0.0).
 *
 * Arguments (-i on rejection):
 *   [1] dtype, [2] layout, [3] n (1..64), [4] nrhs (1..8), [5] batch.
 *   [6] L       device, batch * n * n elements, layout of A; only the
 *               entries on and below the diagonal are read.  Read only.
 *   [7] B       device, read only.
 *   [8] X       device, like B; written; must not overlap L or B.
 *       stream  HIP stream.
 * No status: a zero or non-finite entry of L (other than a failed factor)
 * gives non-finite entries of X.  Ownership, stream semantics and errors as
 * for tdls_gesv_batched.
 */
int tdls_potrs_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                       const void* L, const void* B, void* X, hipStream_t stream);

/*
 * Solve (A_s + shift I) X_s = B_s by Cholesky (LAPACK's posv): the
 * factorization of tdls_potrf_batched with L y = b folded into its steps,
 * then L^T x = y, each x_j = y_j / L(j,j) by IEEE division and removed from
 * the rows above by fused multiply-adds.  Same status, with -1 also for a
 * non-finite entry of B and -3 also for one of y or x; a failed system gets
 * X = +0.0.
 *
 * Arguments (-i on rejection):
 *   [1] dtype, [2] layout, [3] n (1..64), [4] nrhs (1..8), [5] batch.
 *   [6] shift   finite diagonal shift.
 *   [7] A       device, read only.  [8] B  device, read only.
 *   [9] X       device, like B; must not overlap A or B.
 *  [10] info    device, int32 [batch].
 *       stream  HIP stream.
 */
int tdls_posv_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                      double shift, const void* A, const void* B, void* X, int32_t* info,
                      hipStream_t stream);

/* Options of the *_ex calls. */
#define TDLS_SCALE_MAXABS 1u /* flags: whole-matrix max-abs scaling of the LU */

typedef struct tdls_options {
  uint32_t flags;     /* 0, or TDLS_SCALE_MAXABS (gesv and getrf only) */
  uint32_t reserved;  /* must be 0 */
  int64_t interleave; /* W: how the systems of the batch are laid out */
} tdls_options;

/*
 * Batch interleave W of the *_ex calls ("solver_static.hpp File Reference",
 * section Residency: one strided form, element e of a system at
 * base[e * stride], covers arrays of structures (stride 1), structures of
 * arrays (stride = batch) and arrays of structures of arrays (stride = W)).
 * For a per-system array of E elements (A, LU, L: E = n*n in the layout
 * flag's order; B, X: E = n*nrhs; piv: E = n), element e of system s lives
 * at
 *     (s / W) * W * E + (s % W) + e * W.
 * W = 0 or 1: systems one after another, as in the plain calls.  W = batch:
 * a structure of arrays.  1 < W < batch: blocks of W systems; when batch
 * is not a multiple of W the last block still spans W * E elements (its
 * missing systems are neither read nor written).  W must not exceed batch
 * (for batch > 0).  info stays one int32 per system, in order.  Results
 * are bitwise those of the plain calls on the same systems.
 */

/*
 * tdls_gesv_batched with options (opt may be NULL: no options).
 *
 * TDLS_SCALE_MAXABS ("ruSOLVER：小矩阵 kernel 优化（实验性）", section on the
 * unchanged numerical and failure contract: the LU keeps its scaling by
 * the largest absolute value of the whole matrix and restores the scale of
 * U at the end): each system is divided, entry by entry (IEEE division),
 * by s = max |A(r,c)| over its matrix, right-hand sides included, which
 * leaves the solution unchanged; a zero matrix is not scaled.  The status
 * is decided on the scaled system (a non-finite input still gives -1).
 *
 * Arguments: [1]..[5] as for tdls_gesv_batched, [6] opt (-6 for an unknown
 * flag, a nonzero reserved field, or an interleave below 0 or above batch),
 * [7] A, [8] B, [9] X, [10] piv, [11] info, stream.  Buffers span the
 * interleaved extent (see tdls_options).
 */
int tdls_gesv_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                         const tdls_options* opt, const void* A, const void* B, void* X,
                         int32_t* piv, int32_t* info, hipStream_t stream);

/*
 * tdls_getrf_batched with options (opt may be NULL).  With
 * TDLS_SCALE_MAXABS the matrix is divided by its largest magnitude s before
 * the elimination and U is multiplied back by s at the end (its scale
 * restored; L is scale-free); the -3 status covers the restored U.
 *
 * Arguments: [1]..[4] as for tdls_getrf_batched, [5] opt, [6] A, [7] LU,
 * [8] piv, [9] info, stream.
 */
int tdls_getrf_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch,
                          const tdls_options* opt, const void* A, void* LU, int32_t* piv,
                          int32_t* info, hipStream_t stream);

/*
 * tdls_getrs_batched with options (opt may be NULL; no flags): the batch
 * interleave applies to LU, piv, B and X alike.
 *
 * Arguments: [1]..[5] as for tdls_getrs_batched, [6] opt, [7] LU, [8] piv,
 * [9] B, [10] X, stream.
 */
int tdls_getrs_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                          const tdls_options* opt, const void* LU, const int32_t* piv,
                          const void* B, void* X, hipStream_t stream);

/*
 * tdls_potrf_batched with options (opt may be NULL; no flags): the batch
 * interleave applies to A and L.
 *
 * Arguments: [1]..[5] as for tdls_potrf_batched, [6] opt, [7] A, [8] L,
 * [9] info, stream.
 */
int tdls_potrf_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch,
                          double shift, const tdls_options* opt, const void* A, void* L,
                          int32_t* info, hipStream_t stream);

/*
 * tdls_potrs_batched with options (opt may be NULL; no flags): the batch
 * interleave applies to L, B and X.
 *
 * Arguments: [1]..[5] as for tdls_potrs_batched, [6] opt, [7] L, [8] B,
 * [9] X, stream.
 */
int tdls_potrs_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                          const tdls_options* opt, const void* L, const void* B, void* X,
                          hipStream_t stream);

/*
 * tdls_posv_batched with options (opt may be NULL; no flags): the batch
 * interleave applies to A, B and X.
 *
 * Arguments: [1]..[6] as for tdls_posv_batched, [7] opt, [8] A, [9] B,
 * [10] X, [11] info, stream.
 */
int tdls_posv_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                         double shift, const tdls_options* opt, const void* A, const void* B,
                         void* X, int32_t* info, hipStream_t stream);

/*
 * tdls_plan_gesv for any operation: [1] op, then the scalar arguments of
 * tdls_plan_gesv shifted by one ([2] dtype ... [6] batch, [7] out); nrhs is
 * ignored for TDLS_OP_GETRF and TDLS_OP_POTRF.  Host only.
 */
int tdls_plan_op(tdls_op op, tdls_dtype dtype, tdls_layout layout, int n, int nrhs,
                 int64_t batch, tdls_plan* out);

/* Static description of a return code (never NULL). */
const char* tdls_strerror(int code);

/* Library version string, e.g. "tdls-mi355x 0.1.0 gfx950". */
const char* tdls_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TDLS_H */
