"""Seeded synthetic inputs for batched gesv.

This module draws random matrices and right-hand sides and lays them out in
storage order.  It holds none of the solver's arithmetic; the one recipe that
depends on a factorization (redrawing systems whose pivot choice is nearly
tied) takes the function that measures the tie as an argument, so the caller
decides which implementation measures it.

Recipes (numpy ``default_rng(seed)``; every draw is float64 and is rounded to
the working dtype afterwards; draws happen in the order A, then B, then the
recipe's modifications):

  n8_f32_row       n=8,  nrhs=1, batch=1024,      float32, row-major,
                   A, B iid U(-1, 1).
  n16_f32_row_sing n=16, nrhs=4, batch=65536,     float32, row-major,
                   A, B iid U(-1, 1); floor(1% of batch) systems, chosen
                   without replacement, get row 5 := row 0 after rounding to
                   float32 (bitwise-equal rows, so the system is singular).
  n32_f64_col      n=32, nrhs=1, batch=262144,    float64, column-major,
                   A, B iid N(0, 1); any system whose smallest relative
                   pivot-candidate gap is below 1e-9 has its matrix redrawn.
  n24_f32_row_scl  n=24, nrhs=2, batch=1000000,   float32, row-major,
                   A iid U(-1, 1), then row i of each system times 10**u_i,
                   u_i iid U(-3, 3) (in float64, before rounding); B iid
                   U(-1, 1).
  n64_f64_row      n=64, nrhs=8, batch=131072,    float64, row-major,
                   A iid N(0, 1) plus 0.5 on the diagonal; B iid N(0, 1).

Symmetric positive definite recipes for the Cholesky path (the same shapes
as three of the above):

  spd_n16_f32_row  n=16, nrhs=4, batch=65536,  float32, row-major
  spd_n32_f64_col  n=32, nrhs=1, batch=262144, float64, column-major
  spd_n64_f64_row  n=64, nrhs=8, batch=131072, float64, row-major
                   G iid N(0, 1) [batch, n, n], A = G G^T / n + I in
                   float64, rounded to the working dtype and made exactly
                   symmetric (the upper triangle mirrors the lower); B iid
                   N(0, 1), drawn after G.

Every recipe accepts a smaller ``batch`` for quick runs: the draws are then
the first systems of the same kind of stream, not a prefix of the full batch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

__all__ = ["Workload", "RECIPES", "SPD_RECIPES", "make", "logical_to_storage",
           "rhs_logical_to_storage"]


@dataclass(frozen=True)
class Recipe:
    name: str
    n: int
    nrhs: int
    batch: int
    dtype: str          # "f32" | "f64"
    layout: str         # "row" | "col"
    dist: str           # "uniform" | "normal"
    note: str


RECIPES = {
    r.name: r
    for r in (
        Recipe("n8_f32_row", 8, 1, 1024, "f32", "row", "uniform",
               "A, B iid U(-1,1), seed 0"),
        Recipe("n16_f32_row_sing", 16, 4, 65536, "f32", "row", "uniform",
               "A, B iid U(-1,1); 1% of systems get row 5 := row 0"),
        Recipe("n32_f64_col", 32, 1, 262144, "f64", "col", "normal",
               "A, B iid N(0,1); systems with pivot gap < 1e-9 redrawn"),
        Recipe("n24_f32_row_scl", 24, 2, 1000000, "f32", "row", "uniform",
               "A iid U(-1,1), row i scaled by 10**U(-3,3); B iid U(-1,1)"),
        Recipe("n64_f64_row", 64, 8, 131072, "f64", "row", "normal",
               "A iid N(0,1) + 0.5 I; B iid N(0,1)"),
    )
}

SPD_RECIPES = {
    r.name: r
    for r in (
        Recipe("spd_n16_f32_row", 16, 4, 65536, "f32", "row", "normal",
               "A = G G^T / n + I, G iid N(0,1), exactly symmetric; B iid N(0,1)"),
        Recipe("spd_n32_f64_col", 32, 1, 262144, "f64", "col", "normal",
               "A = G G^T / n + I, G iid N(0,1), exactly symmetric; B iid N(0,1)"),
        Recipe("spd_n64_f64_row", 64, 8, 131072, "f64", "row", "normal",
               "A = G G^T / n + I, G iid N(0,1), exactly symmetric; B iid N(0,1)"),
    )
}

GAP_THRESHOLD = 1e-9


@dataclass
class Workload:
    name: str
    n: int
    nrhs: int
    batch: int
    dtype: str
    layout: str
    A: np.ndarray            # storage order, shape [batch, n, n]
    B: np.ndarray            # storage order, [batch, n, nrhs] (row) or [batch, nrhs, n] (col)
    meta: dict = field(default_factory=dict)

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float64


def logical_to_storage(A: np.ndarray, layout: str) -> np.ndarray:
    """[batch, n, n] logical -> contiguous storage of the given layout."""
    return np.ascontiguousarray(A if layout == "row" else A.transpose(0, 2, 1))


def rhs_logical_to_storage(B: np.ndarray, layout: str) -> np.ndarray:
    """[batch, n, nrhs] logical -> contiguous storage of the given layout."""
    return np.ascontiguousarray(B if layout == "row" else B.transpose(0, 2, 1))


def _draw(rng: np.random.Generator, dist: str, shape, chunk_rows: int = 1 << 15) -> np.ndarray:
    """Float64 draws, produced in chunks along axis 0 to bound the peak memory.
    Chunked draws consume the generator in the same order as one big draw."""
    out = np.empty(shape, dtype=np.float64)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        sub = (e - s,) + tuple(shape[1:])
        if dist == "uniform":
            out[s:e] = rng.uniform(-1.0, 1.0, size=sub)
        else:
            out[s:e] = rng.standard_normal(size=sub)
    return out


def make(name: str, seed: int = 0, batch: Optional[int] = None,
         gap_fn: Optional[Callable[[np.ndarray, int, str], np.ndarray]] = None) -> Workload:
    """Build one recipe's inputs.

    ``gap_fn(A_storage, n, layout) -> gaps`` is used only by ``n32_f64_col``:
    systems whose gap is below 1e-9 are redrawn (matrix only) from the same
    stream until none is left.  Without it no system is redrawn, and
    ``meta["gap_filtered"]`` says so.
    """
    if name in SPD_RECIPES:
        return _make_spd(name, seed, batch)
    r = RECIPES[name]
    b = r.batch if batch is None else int(batch)
    n, nrhs = r.n, r.nrhs
    wdt = np.float32 if r.dtype == "f32" else np.float64
    rng = np.random.default_rng(seed)
    meta: dict = {"recipe": r.note, "seed": seed}

    A64 = _draw(rng, r.dist, (b, n, n))
    B64 = _draw(rng, r.dist, (b, n, nrhs))

    if name == "n24_f32_row_scl":
        u = rng.uniform(-3.0, 3.0, size=(b, n))
        A64 *= np.power(10.0, u)[:, :, None]
    if name == "n64_f64_row":
        idx = np.arange(n)
        A64[:, idx, idx] += 0.5

    A = A64.astype(wdt)
    del A64
    B = B64.astype(wdt)
    del B64

    if name == "n16_f32_row_sing":
        count = (b * 1) // 100
        chosen = np.sort(rng.choice(b, size=count, replace=False)) if count > 0 else np.zeros(0, np.int64)
        A[chosen, 5, :] = A[chosen, 0, :]
        meta["singular"] = chosen

    A_st = logical_to_storage(A, r.layout)
    del A
    B_st = rhs_logical_to_storage(B, r.layout)

    if name == "n32_f64_col":
        meta["gap_filtered"] = gap_fn is not None
        redrawn = 0
        if gap_fn is not None:
            bad = np.nonzero(gap_fn(A_st, n, r.layout) < GAP_THRESHOLD)[0]
            rounds = 0
            while bad.size:
                rounds += 1
                if rounds > 100:
                    raise RuntimeError("pivot-gap redraw did not converge")
                fresh = _draw(rng, r.dist, (bad.size, n, n)).astype(wdt)
                A_st[bad] = logical_to_storage(fresh, r.layout)
                redrawn += bad.size
                g = gap_fn(np.ascontiguousarray(A_st[bad]), n, r.layout)
                bad = bad[g < GAP_THRESHOLD]
        meta["redrawn"] = redrawn

    return Workload(name, n, nrhs, b, r.dtype, r.layout, A_st, B_st, meta)


def _make_spd(name: str, seed: int, batch: Optional[int]) -> Workload:
    r = SPD_RECIPES[name]
    b = r.batch if batch is None else int(batch)
    n, nrhs = r.n, r.nrhs
    wdt = np.float32 if r.dtype == "f32" else np.float64
    rng = np.random.default_rng(seed)
    G = _draw(rng, "normal", (b, n, n))
    B = _draw(rng, "normal", (b, n, nrhs)).astype(wdt)
    A = np.empty((b, n, n), dtype=wdt)
    chunk = 1 << 14
    for s0 in range(0, b, chunk):
        g = G[s0:s0 + chunk]
        m = (g @ g.transpose(0, 2, 1)) / n + np.eye(n)
        m = m.astype(wdt)
        low = np.tril(m)
        A[s0:s0 + chunk] = low + np.tril(m, -1).transpose(0, 2, 1)
    del G
    meta = {"recipe": r.note, "seed": seed}
    return Workload(name, n, nrhs, b, r.dtype, r.layout, logical_to_storage(A, r.layout),
                    rhs_logical_to_storage(B, r.layout), meta)
