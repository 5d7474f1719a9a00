/*
 * Body of the CPU oracle, written once and included twice by gesv_oracle.c:
 * once with REAL = double (suffix _f64) and once with REAL = float (suffix _f32).
 * Every operation runs in REAL, the working precision of the system, because
 * the pivot choice and the exact-zero test of the pivot are decisions taken in
 * that precision.
 *
 * TEST INFRASTRUCTURE ONLY.  See gesv_oracle.c for the provenance of each step.
 *
 * Macros expected from the includer:
 *   REAL   element type
 *   SFX(x) appends the suffix (_f64 / _f32) to an identifier
 *   FMA    fused multiply-add of REAL (fma / fmaf)
 *   FABS   absolute value of REAL (fabs / fabsf)
 *   SQRT   square root of REAL, correctly rounded (sqrt / sqrtf)
 */

/* Logical element (r, c) of the matrix of one system, whatever its storage.
 * Row-major: (r, c) at r*n + c.  Column-major: (r, c) at c*n + r. */
static REAL SFX(load_a)(const REAL *a, int layout, int n, int r, int c)
{
    return layout == ORACLE_ROW_MAJOR ? a[(size_t)r * n + c] : a[(size_t)c * n + r];
}

/* Right-hand sides and solutions follow the same layout flag as the matrix:
 * row-major n x nrhs (r, j) at r*nrhs + j, column-major at j*n + r. */
static size_t SFX(rhs_index)(int layout, int n, int nrhs, int r, int j)
{
    return layout == ORACLE_ROW_MAJOR ? (size_t)r * nrhs + j : (size_t)j * n + r;
}

/*
 * Magnitude order of the pivot search: v ranks strictly above m.  Numbers
 * compare as numbers; a NaN ranks above every number (IEEE 754 totalOrder
 * places NaN beyond infinity) and equal to another NaN.  Inputs are finite
 * (a non-finite input fails with status -1 before any step), so a NaN
 * candidate can only be an intermediate result, and the system then fails
 * with status -3 whatever is chosen; the order only has to be total so that
 * the choice, and hence a zero-pivot status, is well defined.
 */
static int SFX(ranks_above)(REAL v, REAL m)
{
    if (isnan(v))
        return !isnan(m);
    return v > m;
}

/*
 * Partial pivoting, first maximum: scan the candidates of column k in
 * increasing current row position, replacing the running choice only when a
 * magnitude ranks strictly above it.  On equal magnitudes the lowest current
 * position therefore wins (LAPACK's choice, the tie rule of the ruSOLVER
 * numerical contract and the first-maximum rule of the SparseDirectSolver
 * review).  Returns the position; *mag receives the winning magnitude.
 */
static int SFX(pivot_search)(const REAL *M, int n, int k, REAL *mag)
{
    int p = k;
    REAL m = FABS(M[(size_t)k * n + k]);
    for (int r = k + 1; r < n; ++r) {
        REAL v = FABS(M[(size_t)r * n + k]);
        if (SFX(ranks_above)(v, m)) {
            p = r;
            m = v;
        }
    }
    *mag = m;
    return p;
}

static void SFX(swap_rows)(REAL *M, int width, int i, int j)
{
    for (int c = 0; c < width; ++c) {
        REAL t = M[(size_t)i * width + c];
        M[(size_t)i * width + c] = M[(size_t)j * width + c];
        M[(size_t)j * width + c] = t;
    }
}

/* 1 when every one of the count values is finite (no NaN, no infinity). */
static int SFX(all_finite)(const REAL *v, size_t count)
{
    for (size_t e = 0; e < count; ++e)
        if (!isfinite(v[e]))
            return 0;
    return 1;
}

/*
 * Whole-matrix max-abs scaling (ruSOLVER page, section on the unchanged
 * numerical and failure contract: the LU keeps its scaling by the largest
 * absolute value of the whole matrix and restores the scale of U at the
 * end).  Reading: the system is scaled as a whole, M / s and Y / s with
 * s = max |M(r,c)| (each entry by IEEE division), which leaves the solution
 * unchanged; a zero matrix (s == 0) is left as it is.  Returns s, or 1 when
 * nothing was scaled.
 */
static REAL SFX(scale_system)(REAL *M, int n, REAL *Y, int nrhs)
{
    REAL s = 0;
    for (size_t e = 0; e < (size_t)n * n; ++e)
        if (FABS(M[e]) > s)
            s = FABS(M[e]);
    if (!(s > 0))
        return (REAL)1;
    for (size_t e = 0; e < (size_t)n * n; ++e)
        M[e] = M[e] / s;
    for (size_t e = 0; e < (size_t)n * nrhs; ++e)
        Y[e] = Y[e] / s;
    return s;
}

/*
 * gesv of one system.  M (n*n) and Y (n*nrhs) are scratch, logical row-major.
 *
 * Right-looking LU with partial row pivoting, P A = L U, with the forward
 * substitution L y = P b carried along with the elimination (each rank-1
 * step also updates the right-hand sides), then U x = y by back substitution
 * taken one solution entry at a time, that entry then eliminated from the
 * rows above it.  This is the order of the cooperative LU solver page
 * (solver_static.hpp, Detailed Description, column-major case) and of its
 * "Departures from the MAGMA kernel" (solution entry kept by its owner).
 *
 * Result contract (ruSOLVER small-matrix page, section on the unchanged
 * numerical and failure contract), in this order of precedence: -1 when an
 * entry of A or B is not finite; k >= 1 for the first pivot that fails
 * (here: an exactly zero pivot, 1-based step); -3 when a computed value is
 * not finite (an entry of L, U, y = L^-1 P b or x); else 0.  A failed
 * system has every solution entry +0.0 and every pivot -1.  With `scale`
 * the system is first scaled by its largest magnitude (scale_system).
 */
static int SFX(gesv_one)(int layout, int n, int nrhs, int scale, const REAL *a, const REAL *b,
                         REAL *x, int32_t *piv, REAL *M, REAL *Y)
{
    for (int r = 0; r < n; ++r)
        for (int c = 0; c < n; ++c)
            M[(size_t)r * n + c] = SFX(load_a)(a, layout, n, r, c);
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)r * nrhs + j] = b[SFX(rhs_index)(layout, n, nrhs, r, j)];

    int info = 0;
    if (!SFX(all_finite)(M, (size_t)n * n) || !SFX(all_finite)(Y, (size_t)n * nrhs))
        info = -1;
    else if (scale)
        (void)SFX(scale_system)(M, n, Y, nrhs);
    for (int k = 0; k < n && info == 0; ++k) {
        REAL mag;
        int p = SFX(pivot_search)(M, n, k, &mag);
        piv[k] = p;
        if (mag == 0) { /* exactly zero pivot: the first failure decides */
            info = k + 1;
            break;
        }
        if (p != k) {
            SFX(swap_rows)(M, n, k, p);
            SFX(swap_rows)(Y, nrhs, k, p);
        }
        const REAL d = M[(size_t)k * n + k];
        for (int r = k + 1; r < n; ++r) {
            /* multiplier by correctly rounded IEEE division (no reciprocal) */
            const REAL l = M[(size_t)r * n + k] / d;
            M[(size_t)r * n + k] = l;
            for (int c = k + 1; c < n; ++c)
                M[(size_t)r * n + c] = FMA(-l, M[(size_t)k * n + c], M[(size_t)r * n + c]);
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)r * nrhs + j] = FMA(-l, Y[(size_t)k * nrhs + j], Y[(size_t)r * nrhs + j]);
        }
    }

    if (info == 0 &&
        (!SFX(all_finite)(M, (size_t)n * n) || !SFX(all_finite)(Y, (size_t)n * nrhs)))
        info = -3; /* L, U or y */

    if (info == 0) {
        /* U x = y: x_k = y_k / u_kk, then x_k leaves the rows r < k. */
        for (int k = n - 1; k >= 0; --k) {
            const REAL ukk = M[(size_t)k * n + k];
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / ukk;
            for (int r = 0; r < k; ++r)
                for (int j = 0; j < nrhs; ++j)
                    Y[(size_t)r * nrhs + j] =
                        FMA(-M[(size_t)r * n + k], Y[(size_t)k * nrhs + j], Y[(size_t)r * nrhs + j]);
        }
        if (!SFX(all_finite)(Y, (size_t)n * nrhs))
            info = -3; /* x */
    }

    if (info != 0) {
        for (int r = 0; r < n; ++r) {
            piv[r] = -1;
            for (int j = 0; j < nrhs; ++j)
                x[SFX(rhs_index)(layout, n, nrhs, r, j)] = (REAL)0;
        }
        return info;
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            x[SFX(rhs_index)(layout, n, nrhs, r, j)] = Y[(size_t)r * nrhs + j];
    return 0;
}

/*
 * getrf of one system: the same elimination, but it records the factors and
 * does not stop at a zero pivot, so that P A = L U can be rebuilt for every
 * input (a zero pivot column gets zero multipliers: all its candidates are
 * zero already).  lu (n*n, logical row-major) receives L strictly below the
 * diagonal (unit diagonal implied) and U on and above it, in LAPACK's
 * pivoted row order; ipiv[k] is the 0-based position swapped with k at step k.
 *
 * *gap receives the smallest, over the steps k <= n-2, relative distance
 * (|c1| - |c2|) / |c1| between the two largest candidate magnitudes of the
 * step (0 when the largest is 0; 1 when n == 1).  A small gap marks a pivot
 * choice that rounding could flip.
 *
 * Status as in gesv_one: -1 for a non-finite entry of A (lu then all +0.0,
 * ipiv all -1, gap 0), the first zero pivot, then -3 when an entry of L or U
 * is not finite.  With `scale`, the matrix is divided by its largest
 * magnitude first and U is multiplied back by it at the end (the scale of U
 * restored; L is scale-free).
 */
static int SFX(getrf_one)(int layout, int n, int scale, const REAL *a, REAL *lu, int32_t *ipiv,
                          double *gap)
{
    for (int r = 0; r < n; ++r)
        for (int c = 0; c < n; ++c)
            lu[(size_t)r * n + c] = SFX(load_a)(a, layout, n, r, c);
    if (!SFX(all_finite)(lu, (size_t)n * n)) {
        for (int r = 0; r < n; ++r) {
            ipiv[r] = -1;
            for (int c = 0; c < n; ++c)
                lu[(size_t)r * n + c] = 0;
        }
        *gap = 0.0;
        return -1;
    }
    const REAL sc = scale ? SFX(scale_system)(lu, n, NULL, 0) : (REAL)1;

    int info = 0;
    double g = 1.0;
    for (int k = 0; k < n; ++k) {
        REAL mag;
        int p = SFX(pivot_search)(lu, n, k, &mag);
        ipiv[k] = p;
        if (k <= n - 2) {
            /* second largest candidate magnitude of column k */
            REAL second = 0;
            for (int r = k; r < n; ++r) {
                if (r == p)
                    continue;
                REAL v = FABS(lu[(size_t)r * n + k]);
                if (v > second)
                    second = v;
            }
            double gk = mag == 0 ? 0.0 : ((double)mag - (double)second) / (double)mag;
            if (gk < g)
                g = gk;
        }
        if (mag == 0) {
            if (info == 0)
                info = k + 1;
            for (int r = k + 1; r < n; ++r)
                lu[(size_t)r * n + k] = 0;
            continue;
        }
        if (p != k)
            SFX(swap_rows)(lu, n, k, p);
        const REAL d = lu[(size_t)k * n + k];
        for (int r = k + 1; r < n; ++r) {
            const REAL l = lu[(size_t)r * n + k] / d;
            lu[(size_t)r * n + k] = l;
            for (int c = k + 1; c < n; ++c)
                lu[(size_t)r * n + c] = FMA(-l, lu[(size_t)k * n + c], lu[(size_t)r * n + c]);
        }
    }
    if (scale)
        for (int r = 0; r < n; ++r)
            for (int c = r; c < n; ++c)
                lu[(size_t)r * n + c] = lu[(size_t)r * n + c] * sc;
    if (info == 0 && !SFX(all_finite)(lu, (size_t)n * n))
        info = -3;
    *gap = g;
    return info;
}

/*
 * getrs of one system: solve A x = b from the factors getrf writes (LAPACK's
 * row order: L's multipliers strictly below the diagonal, unit diagonal
 * implied, U on and above it), in the storage layout of the call.  The
 * right-hand sides take the swaps of the sequence one after the other,
 * then L y = P b is solved column by column (y_k leaves the rows below it),
 * then U x = y exactly as in gesv_one.  This is the factor-then-solve split
 * of the same elimination ("solver_static.hpp File Reference", Factored
 * format and Detailed Description), so every entry sees the same fused
 * multiply-adds in the same order as in gesv_one.  A failed factorization
 * (ipiv[0] < 0, every pivot -1 by the ruSOLVER contract) gives x = +0.0.
 */
static void SFX(getrs_one)(int layout, int n, int nrhs, const REAL *lu, const int32_t *ipiv,
                           const REAL *b, REAL *x, REAL *Y)
{
    if (ipiv[0] < 0) {
        for (int r = 0; r < n; ++r)
            for (int j = 0; j < nrhs; ++j)
                x[SFX(rhs_index)(layout, n, nrhs, r, j)] = (REAL)0;
        return;
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)r * nrhs + j] = b[SFX(rhs_index)(layout, n, nrhs, r, j)];
    for (int k = 0; k < n; ++k)
        if (ipiv[k] != k)
            SFX(swap_rows)(Y, nrhs, k, ipiv[k]);
    for (int k = 0; k < n; ++k)
        for (int r = k + 1; r < n; ++r) {
            const REAL l = SFX(load_a)(lu, layout, n, r, k);
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)r * nrhs + j] = FMA(-l, Y[(size_t)k * nrhs + j], Y[(size_t)r * nrhs + j]);
        }
    for (int k = n - 1; k >= 0; --k) {
        const REAL ukk = SFX(load_a)(lu, layout, n, k, k);
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / ukk;
        for (int r = 0; r < k; ++r) {
            const REAL u = SFX(load_a)(lu, layout, n, r, k);
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)r * nrhs + j] = FMA(-u, Y[(size_t)k * nrhs + j], Y[(size_t)r * nrhs + j]);
        }
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            x[SFX(rhs_index)(layout, n, nrhs, r, j)] = Y[(size_t)r * nrhs + j];
}

int SFX(oracle_getrs)(int layout, int n, int nrhs, int64_t batch, const REAL *LU,
                      const int32_t *ipiv, const REAL *B, REAL *X, int nthreads)
{
    int rc = oracle_check_args(layout, n, nrhs, batch);
    if (rc != 0)
        return rc;
    if (batch == 0)
        return 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    for (int64_t s = 0; s < batch; ++s)
        for (int k = 0; k < n; ++k) {
            const int32_t p = ipiv[s * (int64_t)n + k];
            if (ipiv[s * (int64_t)n] >= 0 && (p < k || p >= n))
                return ORACLE_EINVAL; /* not a swap sequence */
        }
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        REAL *Y = (REAL *)malloc(sizeof(REAL) * (size_t)n * nrhs);
        if (Y == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t s = 0; s < batch; ++s)
                SFX(getrs_one)(layout, n, nrhs, LU + s * (int64_t)n * n, ipiv + s * (int64_t)n,
                               B + s * (int64_t)n * nrhs, X + s * (int64_t)n * nrhs, Y);
        }
        free(Y);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

/*
 * Cholesky of one system, A + shift I = L L^T, then (posv) L y = b and
 * L^T x = y.  L is lower triangular, logical row-major n*n, zero above the
 * diagonal.
 *
 * Contract ("ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
 * numerical and failure contract; "cuSolverDx potrf" function page):
 *  - the input must be exactly symmetric, A(i,j) == A(j,i) in the working
 *    precision, else status -2;
 *  - the diagonal shift is explicit: s = A(j,j) + shift, rounded once, and
 *    nothing else is added;
 *  - inner products accumulate in increasing k: s = fma(-L(j,k), L(j,k), s)
 *    for k = 0, 1, ..., j-1, then L(j,j) = sqrt(s) (IEEE square root), and
 *    t = A(i,j), t = fma(-L(i,k), L(j,k), t) for k < j, L(i,j) = t / L(j,j)
 *    (IEEE division) for i > j;
 *  - status j+1 (1-based) for the first step whose s is not > 0 (the
 *    smallest leading minor that is not positive definite, as cuSolverDx
 *    reports it); a failed system (any nonzero status) gets L = +0.0 and
 *    x = +0.0 everywhere;
 *  - precedence of the statuses: -1 for a non-finite input entry (A, and B
 *    for posv), then -2, then j+1, then -3 when a computed value (an entry
 *    of L, y or x) is not finite.
 * The lower triangle is read; the symmetry check makes the choice moot.
 *
 * The solves: y_i = b_i - sum_{k<i} L(i,k) y_k in increasing k, then
 * y_i / L(i,i) (each y_k leaves the rows below it before the next one is
 * formed), and x_j = y_j / L(j,j) for j = n-1 .. 0, each x_j then removed
 * from the rows above it: y_i = fma(-L(j,i), x_j, y_i).
 */
static int SFX(potrf_one)(int layout, int n, REAL shift, const REAL *a, REAL *L)
{
    if (!SFX(all_finite)(a, (size_t)n * n))
        return -1;
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < i; ++j)
            if (!(SFX(load_a)(a, layout, n, i, j) == SFX(load_a)(a, layout, n, j, i)))
                return -2;
    for (size_t e = 0; e < (size_t)n * n; ++e)
        L[e] = 0;
    for (int j = 0; j < n; ++j) {
        REAL s = SFX(load_a)(a, layout, n, j, j) + shift;
        for (int k = 0; k < j; ++k)
            s = FMA(-L[(size_t)j * n + k], L[(size_t)j * n + k], s);
        if (!(s > 0))
            return j + 1;
        const REAL d = SQRT(s);
        L[(size_t)j * n + j] = d;
        for (int i = j + 1; i < n; ++i) {
            REAL t = SFX(load_a)(a, layout, n, i, j);
            for (int k = 0; k < j; ++k)
                t = FMA(-L[(size_t)i * n + k], L[(size_t)j * n + k], t);
            L[(size_t)i * n + j] = t / d;
        }
    }
    return SFX(all_finite)(L, (size_t)n * n) ? 0 : -3;
}

static void SFX(zero_rhs)(int layout, int n, int nrhs, REAL *x)
{
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            x[SFX(rhs_index)(layout, n, nrhs, r, j)] = (REAL)0;
}

static int SFX(posv_one)(int layout, int n, int nrhs, REAL shift, const REAL *a, const REAL *b,
                         REAL *x, REAL *L, REAL *Y)
{
    int info = SFX(all_finite)(b, (size_t)n * nrhs) ? SFX(potrf_one)(layout, n, shift, a, L) : -1;
    if (info != 0) {
        SFX(zero_rhs)(layout, n, nrhs, x);
        return info;
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)r * nrhs + j] = b[SFX(rhs_index)(layout, n, nrhs, r, j)];
    /* L y = b */
    for (int k = 0; k < n; ++k) {
        const REAL d = L[(size_t)k * n + k];
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / d;
        for (int i = k + 1; i < n; ++i)
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)i * nrhs + j] =
                    FMA(-L[(size_t)i * n + k], Y[(size_t)k * nrhs + j], Y[(size_t)i * nrhs + j]);
    }
    if (!SFX(all_finite)(Y, (size_t)n * nrhs)) {
        SFX(zero_rhs)(layout, n, nrhs, x); /* y */
        return -3;
    }
    /* L^T x = y */
    for (int k = n - 1; k >= 0; --k) {
        const REAL d = L[(size_t)k * n + k];
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / d;
        for (int i = 0; i < k; ++i)
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)i * nrhs + j] =
                    FMA(-L[(size_t)k * n + i], Y[(size_t)k * nrhs + j], Y[(size_t)i * nrhs + j]);
    }
    if (!SFX(all_finite)(Y, (size_t)n * nrhs)) {
        SFX(zero_rhs)(layout, n, nrhs, x); /* x */
        return -3;
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            x[SFX(rhs_index)(layout, n, nrhs, r, j)] = Y[(size_t)r * nrhs + j];
    return 0;
}

int SFX(oracle_potrf)(int layout, int n, int64_t batch, double shift, const REAL *A, REAL *Lout,
                      int32_t *info, int nthreads)
{
    int rc = oracle_check_args(layout, n, 1, batch);
    if (rc != 0)
        return rc;
    if (batch == 0)
        return 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t s = 0; s < batch; ++s) {
        REAL *Ls = Lout + s * (int64_t)n * n;   /* logical row-major */
        info[s] = SFX(potrf_one)(layout, n, (REAL)shift, A + s * (int64_t)n * n, Ls);
        if (info[s] != 0)
            for (size_t e = 0; e < (size_t)n * n; ++e)
                Ls[e] = 0;
    }
    return 0;
}

/*
 * potrs of one system: X from the Cholesky factor that potrf writes (L on
 * and below the diagonal, in the layout of A; the entries above it are not
 * read), by L y = b and L^T x = y in exactly the order of posv_one, so
 * potrf then potrs gives posv's solution.  A failed factorization leaves L
 * all +0.0 (ruSOLVER contract), so L(0,0) == 0 marks it, and x = +0.0.
 * There is no status: a zero or non-finite factor entry flows into x.
 */
static void SFX(potrs_one)(int layout, int n, int nrhs, const REAL *l, const REAL *b, REAL *x,
                           REAL *Y)
{
    if (SFX(load_a)(l, layout, n, 0, 0) == 0) {
        SFX(zero_rhs)(layout, n, nrhs, x);
        return;
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)r * nrhs + j] = b[SFX(rhs_index)(layout, n, nrhs, r, j)];
    /* L y = b: y_k = y_k / L(k,k), then y_k leaves the rows below */
    for (int k = 0; k < n; ++k) {
        const REAL d = SFX(load_a)(l, layout, n, k, k);
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / d;
        for (int i = k + 1; i < n; ++i) {
            const REAL lik = SFX(load_a)(l, layout, n, i, k);
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)i * nrhs + j] = FMA(-lik, Y[(size_t)k * nrhs + j], Y[(size_t)i * nrhs + j]);
        }
    }
    /* L^T x = y: x_k = y_k / L(k,k), then x_k leaves the rows above with L(k,i) */
    for (int k = n - 1; k >= 0; --k) {
        const REAL d = SFX(load_a)(l, layout, n, k, k);
        for (int j = 0; j < nrhs; ++j)
            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / d;
        for (int i = 0; i < k; ++i) {
            const REAL lki = SFX(load_a)(l, layout, n, k, i);
            for (int j = 0; j < nrhs; ++j)
                Y[(size_t)i * nrhs + j] = FMA(-lki, Y[(size_t)k * nrhs + j], Y[(size_t)i * nrhs + j]);
        }
    }
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < nrhs; ++j)
            x[SFX(rhs_index)(layout, n, nrhs, r, j)] = Y[(size_t)r * nrhs + j];
}

int SFX(oracle_potrs)(int layout, int n, int nrhs, int64_t batch, const REAL *L, const REAL *B,
                      REAL *X, int nthreads)
{
    int rc = oracle_check_args(layout, n, nrhs, batch);
    if (rc != 0)
        return rc;
    if (batch == 0)
        return 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        REAL *Y = (REAL *)malloc(sizeof(REAL) * (size_t)n * nrhs);
        if (Y == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t s = 0; s < batch; ++s)
                SFX(potrs_one)(layout, n, nrhs, L + s * (int64_t)n * n, B + s * (int64_t)n * nrhs,
                               X + s * (int64_t)n * nrhs, Y);
        }
        free(Y);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

int SFX(oracle_posv)(int layout, int n, int nrhs, int64_t batch, double shift, const REAL *A,
                     const REAL *B, REAL *X, int32_t *info, int nthreads)
{
    int rc = oracle_check_args(layout, n, nrhs, batch);
    if (rc != 0)
        return rc;
    if (batch == 0)
        return 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        REAL *L = (REAL *)malloc(sizeof(REAL) * (size_t)n * n);
        REAL *Y = (REAL *)malloc(sizeof(REAL) * (size_t)n * nrhs);
        if (L == NULL || Y == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t s = 0; s < batch; ++s)
                info[s] = SFX(posv_one)(layout, n, nrhs, (REAL)shift, A + s * (int64_t)n * n,
                                        B + s * (int64_t)n * nrhs, X + s * (int64_t)n * nrhs, L,
                                        Y);
        }
        free(L);
        free(Y);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

int SFX(oracle_gesv)(int layout, int n, int nrhs, int64_t batch, int scale, const REAL *A,
                     const REAL *B, REAL *X, int32_t *piv, int32_t *info, int nthreads)
{
    int rc = oracle_check_args(layout, n, nrhs, batch);
    if (rc != 0)
        return rc;
    if (batch == 0)
        return 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        REAL *M = (REAL *)malloc(sizeof(REAL) * (size_t)n * n);
        REAL *Y = (REAL *)malloc(sizeof(REAL) * (size_t)n * nrhs);
        if (M == NULL || Y == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t s = 0; s < batch; ++s) {
                info[s] = SFX(gesv_one)(layout, n, nrhs, scale, A + s * (int64_t)n * n,
                                        B + s * (int64_t)n * nrhs, X + s * (int64_t)n * nrhs,
                                        piv + s * (int64_t)n, M, Y);
            }
        }
        free(M);
        free(Y);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

int SFX(oracle_getrf)(int layout, int n, int64_t batch, int scale, const REAL *A, REAL *LU,
                      int32_t *ipiv, int32_t *info, double *gap, int nthreads)
{
    int rc = oracle_check_args(layout, n, 1, batch);
    if (rc != 0)
        return rc;
    if (batch == 0)
        return 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t s = 0; s < batch; ++s) {
        info[s] = SFX(getrf_one)(layout, n, scale, A + s * (int64_t)n * n,
                                 LU + s * (int64_t)n * n, ipiv + s * (int64_t)n, gap + s);
    }
    return 0;
}
