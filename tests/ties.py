"""Inputs whose pivot choices are decided by exact magnitude ties, and a
replay that says which kinds of tie they exercise.

The tie rule under test: among candidates of equal magnitude the lowest
current row position wins ("ruSOLVER：小矩阵 kernel 优化（实验性）", section on
the unchanged numerical and failure contract: ties to the lowest row number;
LAPACK's first maximum).  A GPU kernel that holds rows tx, tx+T, ... on lane
tx of a T-lane group (rows put back in position order at each multiple of
T, where the kernel compacts its slots) meets ties between two slots of one
lane, between lanes, and ties where the lower position sits on the higher
lane; in float64 also candidates whose high 32-bit words agree and whose low
words decide.  These generators make such ties happen in non-singular
systems, where the choice shows in piv.

Two constructions (numpy ``default_rng(seed)``; nothing here solves):

  dyadic_plu   A = P^T L U with L unit lower triangular, entries drawn from
               {0, +-1/2, +-1} (a +-1 multiplier makes a candidate as large as
               the pivot: an exact tie), U upper triangular with small integer
               entries and a non-zero diagonal, P a random permutation.  Every
               entry of A is a multiple of 1/2 below 2^8 in magnitude, so A is
               exact in float32 and float64, and the eliminations stay on
               short dyadic numbers: the ties survive rounding.
  planted_tie  k "pivot rows" carry a diagonal block (4 on their own column,
               0 elsewhere left of column k) so that steps 0..k-1 take them in
               turn with zero multipliers for every other row; the other rows
               are zero left of column k, so column k reaches step k
               unchanged.  Column k of those rows gets planted values: in
               float64 v = 1 + 2^-40 twice (once negated: a tie) and
               1 + 2^-45 (the same high word, a smaller low word); in float32
               +-v with v = 1 + 2^-20 and 1 (a smaller value).  The rest is
               U(-1/2, 1/2) in column k and U(-1, 1) right of it.

``replay_ties`` repeats the elimination in float64 numpy (valid where the
arithmetic is exact, which ``replay_ties`` checks against the pivots of the
caller) and lists, per step, the positions that tie for the maximum, with
the lane and slot each row occupies in the kernel's layout.
"""
from __future__ import annotations

import numpy as np


def dyadic_plu(rng: np.random.Generator, batch: int, n: int, p_one: float = 0.4,
               p_half: float = 0.3) -> np.ndarray:
    """[batch, n, n] float64 logical matrices A = P^T L U (see the module)."""
    u = rng.random((batch, n, n))
    mag = np.where(u < p_one, 1.0, np.where(u < p_one + p_half, 0.5, 0.0))
    sgn = np.where(rng.random((batch, n, n)) < 0.5, -1.0, 1.0)
    L = np.tril(mag * sgn, -1) + np.eye(n)
    U = np.triu(rng.integers(-2, 3, (batch, n, n)).astype(np.float64), 1)
    d = rng.integers(1, 3, (batch, n)) * np.where(rng.random((batch, n)) < 0.5, -1, 1)
    U += d[:, :, None] * np.eye(n)
    A = np.matmul(L, U)
    perm = np.argsort(rng.random((batch, n)), axis=1)
    return np.take_along_axis(A, perm[:, :, None], axis=1)


def planted_tie(rng: np.random.Generator, batch: int, n: int, k: int, dtype) -> np.ndarray:
    """[batch, n, n] float64 logical matrices with an exact tie planted at
    step k (see the module); ``dtype`` picks the planted values."""
    if not 0 <= k <= n - 3:
        raise ValueError("k must leave three candidates")
    A = np.zeros((batch, n, n))
    for s in range(batch):
        rows = rng.permutation(n)
        piv_rows, rest = rows[:k], rows[k:]
        for i, r in enumerate(piv_rows):
            A[s, r, i] = 4.0
            A[s, r, k:] = rng.uniform(-1, 1, n - k)
        A[s, rest, k] = rng.uniform(-0.5, 0.5, len(rest))
        A[s, rest[:, None], np.arange(k + 1, n)[None, :]] = rng.uniform(-1, 1,
                                                                        (len(rest), n - k - 1))
        t = rng.permutation(rest)[:3]
        if np.dtype(dtype) == np.float64:
            v, w = 1.0 + 2.0 ** -40, 1.0 + 2.0 ** -45
        else:
            v, w = 1.0 + 2.0 ** -20, 1.0
        A[s, t[0], k] = v
        A[s, t[1], k] = -v
        A[s, t[2], k] = w
    return A


def slot_homes(n: int, T: int, compact: bool):
    """Steps at which rows are put back in position order (multiples of T
    below n when the kernel compacts)."""
    return [k0 for k0 in range(T, n, T)] if compact else []


def replay_ties(A: np.ndarray, T: int, compact: bool, piv_expect: np.ndarray,
                is64: bool = True):
    """Elimination with first-maximum pivoting in float64 numpy on logical
    [batch, n, n] matrices.  Returns (events, agree): ``agree`` marks the
    systems whose replayed pivots equal ``piv_expect`` (the oracle's); for
    those, ``events`` lists (system, step, the positions tied for the largest
    magnitude, their lanes, their slots, whether other candidates share the
    largest high word with a smaller low word) for every step where two or
    more candidates tie for the largest magnitude, or where, in float64, the
    largest high word is shared by candidates with different low words."""
    A = np.array(A, dtype=np.float64, copy=True)
    batch, n, _ = A.shape
    pos_row = np.tile(np.arange(n), (batch, 1))      # position -> original row
    home = np.tile(np.arange(n), (batch, 1))         # original row -> home index
    boundaries = set(slot_homes(n, T, compact))
    piv = np.zeros((batch, n), np.int64)
    raw = []
    M = A.copy()                                     # rows in position order
    for k in range(n):
        if k in boundaries:
            for s in range(batch):
                home[s, pos_row[s]] = np.arange(n)
        col = np.abs(M[:, k:, k])
        mx = col.max(axis=1)
        tied = col == mx[:, None]
        if is64:   # the kernel compares float64 magnitudes by high word first
            hi = np.ascontiguousarray(col).view(np.uint64) >> np.uint64(32)
            hi_tied = hi == hi.max(axis=1)[:, None]
        else:
            hi_tied = tied
        p = k + np.argmax(col, axis=1)
        piv[:, k] = p
        for s in np.nonzero((tied.sum(axis=1) > 1) | (hi_tied.sum(axis=1) > tied.sum(axis=1)))[0]:
            cand = k + np.nonzero(tied[s])[0]
            rows = pos_row[s, cand]
            raw.append((int(s), k, cand.tolist(), (home[s, rows] % T).tolist(),
                        (home[s, rows] // T).tolist(), bool(hi_tied[s].sum() > tied[s].sum())))
        rs = np.arange(batch)
        Mk, Mp = M[rs, k].copy(), M[rs, p].copy()
        M[rs, k], M[rs, p] = Mp, Mk
        rk, rp = pos_row[rs, k].copy(), pos_row[rs, p].copy()
        pos_row[rs, k], pos_row[rs, p] = rp, rk
        d = M[:, k, k]
        safe = np.where(d == 0, 1.0, d)
        l = M[:, k + 1:, k] / safe[:, None]
        M[:, k + 1:, k + 1:] -= l[:, :, None] * M[:, k, None, k + 1:]
        M[:, k + 1:, k] = l
    agree = (piv == piv_expect).all(axis=1)
    events = [e for e in raw if agree[e[0]]]
    return events, agree


def classify(events) -> dict:
    """Counts of the tie kinds among replayed events: a tie of exactly equal
    magnitudes between two slots of one lane, across lanes, with the winner
    (lowest position) on a higher lane than another tied row, and float64
    candidates sharing the largest high word with different low words."""
    out = {"same_lane_two_slots": 0, "across_lanes": 0, "lower_position_higher_lane": 0,
           "equal_high_word": 0, "events": len(events)}
    for _, _, cand, lanes, slots, hi_only in events:
        if hi_only:
            out["equal_high_word"] += 1
        w = 0  # cand is sorted: the lowest position is first
        for j in range(1, len(cand)):
            if lanes[j] == lanes[w] and slots[j] != slots[w]:
                out["same_lane_two_slots"] += 1
            if lanes[j] != lanes[w]:
                out["across_lanes"] += 1
            if lanes[w] > lanes[j]:
                out["lower_position_higher_lane"] += 1
    return out


# Shapes of the tie tests: (n, dtype, nrhs), the benchmark's right-hand-side
# counts where a recipe has this n.
SHAPES = [(16, "f32", 4), (16, "f64", 4), (24, "f32", 2), (24, "f64", 2), (32, "f32", 1),
          (32, "f64", 1), (48, "f32", 3), (48, "f64", 3), (64, "f32", 8), (64, "f64", 8)]


def tie_batch(n: int, dtype: str, seed: int = 0):
    """Logical A [batch, n, n] and B [batch, n, nrhs-free: 1 column per call
    site] in the working dtype: 300 dyadic P^T L U systems, then 20 planted
    ties at each of the steps 0, 1, 3, T-1, T, T+1 for T in {4, 16} and
    n - 3 (those that leave three candidates)."""
    npdt = np.float32 if dtype == "f32" else np.float64
    rng = np.random.default_rng(seed + 1000 * n + (7 if dtype == "f64" else 0))
    parts = [dyadic_plu(rng, 300, n)]
    for k in sorted({0, 1, 3, 15, 16, 17, n - 3}):
        if k <= n - 3:
            parts.append(planted_tie(rng, 20, n, k, npdt))
    return np.concatenate(parts).astype(npdt)
