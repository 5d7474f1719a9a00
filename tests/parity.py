"""Comparison of the GPU library with the oracle, shared by the GPU tests
and the smoke check.

The bar (element by element, same seeded inputs):
  * info: bit-exact.
  * piv: bit-exact on systems whose pivot gap (oracle, working precision)
    leaves no room for rounding to flip a choice: >= 1e-9 (float64) or
    >= 1e-4 (float32).  Mismatches elsewhere are counted, not failed.
  * X: normwise relative error vs the oracle <= 1e-4 (float32) or <= 1e-11
    (float64) on systems with kappa_inf <= 1e3 (a system above the
    tolerance passes only if it is worse conditioned than that).
  * scaled residual ||Ax - b|| / (n eps ||A|| ||x||) <= 10 on every
    non-singular system.
  * failed systems: X all +0.0 and piv all -1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import metrics
import oracle

X_TOL = {np.dtype(np.float32): 1e-4, np.dtype(np.float64): 1e-11}
GAP_TOL = {np.dtype(np.float32): 1e-4, np.dtype(np.float64): 1e-9}
RESID_TOL = 10.0
KAPPA_MAX = 1e3


@dataclass
class Report:
    systems: int
    info_mismatch: int
    piv_checked: int
    piv_mismatch_margin: int
    piv_mismatch_nomargin: int
    x_checked: int
    x_max_err: float
    resid_checked: int
    resid_max: float
    failed_bad_outputs: int
    bitwise_x_equal: int
    notes: list = field(default_factory=list)

    def ok(self) -> bool:
        return (self.info_mismatch == 0 and self.piv_mismatch_margin == 0
                and self.failed_bad_outputs == 0
                and (self.x_checked == 0 or self.x_max_err <= self.x_tol)
                and (self.resid_checked == 0 or self.resid_max <= RESID_TOL))

    x_tol: float = 0.0


def compare(A_st: np.ndarray, B_st: np.ndarray, X_st: np.ndarray, piv: np.ndarray,
            info: np.ndarray, n: int, nrhs: int, layout: str, idx=None,
            scale: bool = False, piv_all: bool = False) -> Report:
    """Compare GPU outputs with the oracle on the systems ``idx`` (all by
    default).  Arrays are host copies in storage order.  ``scale``: the
    outputs come from the max-abs scaled solve.  ``piv_all``: piv must equal
    the oracle's on every system, whatever its pivot gap (inputs built so
    that exact ties, not rounding, decide the pivots)."""
    dt = np.dtype(A_st.dtype)
    A_st = A_st.reshape(-1, n * n)
    B_st = B_st.reshape(-1, n * nrhs)
    X_st = X_st.reshape(-1, n * nrhs)
    piv = piv.reshape(-1, n)
    info = info.reshape(-1)
    if idx is not None:
        idx = np.asarray(idx)
        A_st, B_st, X_st, piv, info = A_st[idx], B_st[idx], X_st[idx], piv[idx], info[idx]
    A_st = np.ascontiguousarray(A_st)
    B_st = np.ascontiguousarray(B_st)
    Xo, pivo, infoo = oracle.gesv(A_st, B_st, n, nrhs, layout, scale=scale)
    _, _, _, gap = oracle.getrf(A_st, n, layout, scale=scale)

    A = oracle.from_storage(A_st, layout, n)
    B = oracle.rhs_from_storage(B_st, layout, n, nrhs)
    X = oracle.rhs_from_storage(X_st, layout, n, nrhs)
    Xr = oracle.rhs_from_storage(Xo, layout, n, nrhs)

    info_mm = int((info != infoo).sum())
    ok_sys = (infoo == 0) & (info == 0)
    margin = gap >= GAP_TOL[dt]
    piv_eq = (piv == pivo).all(axis=1)
    rep_piv_checked = int((margin & ok_sys).sum())
    if piv_all:
        margin = np.ones_like(margin)
        rep_piv_checked = int(ok_sys.sum())
    piv_mm_margin = int((~piv_eq & margin).sum())
    piv_mm_nomargin = int((~piv_eq & ~margin).sum())

    failed = infoo != 0
    bad_failed = 0
    if failed.any():
        Xf = X_st[failed]
        bad_failed = int(((Xf != 0) | np.signbit(Xf)).any(axis=1).sum()
                         + (piv[failed] != -1).any(axis=1).sum())

    # The X bar holds where kappa_inf <= 1e3.  Every solved system's error
    # is measured; kappa is computed only for those above the tolerance
    # (exempt when ill-conditioned), so a full batch needs no million
    # inversions.  x_checked counts the systems held to the bar.
    err = metrics.normwise_error(X[ok_sys], Xr[ok_sys]) if ok_sys.any() else np.zeros(0)
    over = err > X_TOL[dt]
    held = np.ones(err.shape, bool)
    if over.any():
        held[over] = metrics.kappa_inf(A[ok_sys][over]) <= KAPPA_MAX
    x_max = float(err[held].max()) if held.any() else 0.0
    res = metrics.residual_ratio(A[ok_sys], X[ok_sys], B[ok_sys], dt) if ok_sys.any() else np.zeros(0)
    bitwise = int((X_st[ok_sys] == Xo.reshape(-1, n * nrhs)[ok_sys]).all(axis=1).sum())

    rep = Report(systems=int(len(info)), info_mismatch=info_mm, piv_checked=rep_piv_checked,
                 piv_mismatch_margin=piv_mm_margin, piv_mismatch_nomargin=piv_mm_nomargin,
                 x_checked=int(held.sum()), x_max_err=x_max, resid_checked=int(len(res)),
                 resid_max=float(res.max()) if len(res) else 0.0, failed_bad_outputs=bad_failed,
                 bitwise_x_equal=bitwise)
    rep.x_tol = X_TOL[dt]
    return rep


def compare_chunked(A_st, B_st, X_st, piv, info, n: int, nrhs: int, layout: str, idx=None,
                    chunk: int = 0, **kw) -> Report:
    """``compare`` over the systems ``idx`` (all by default) in chunks, so
    that a whole full-size batch can be checked against the oracle with
    bounded host memory; counts add up, maxima combine."""
    batch = np.asarray(info).reshape(-1).shape[0]
    idx = np.arange(batch) if idx is None else np.asarray(idx)
    chunk = chunk or max(1024, (1 << 24) // (n * n))
    out = None
    for s in range(0, len(idx), chunk):
        r = compare(A_st, B_st, X_st, piv, info, n, nrhs, layout, idx=idx[s:s + chunk], **kw)
        if out is None:
            out = r
            continue
        for f in ("systems", "info_mismatch", "piv_checked", "piv_mismatch_margin",
                  "piv_mismatch_nomargin", "x_checked", "resid_checked", "failed_bad_outputs",
                  "bitwise_x_equal"):
            setattr(out, f, getattr(out, f) + getattr(r, f))
        out.x_max_err = max(out.x_max_err, r.x_max_err)
        out.resid_max = max(out.resid_max, r.resid_max)
    return out
