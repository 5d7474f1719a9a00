"""The tie inputs (tests/ties.py) are what the GPU tie tests need: every
system is non-singular, its pivots are decided by exact ties, and together
they put tied candidates in every arrangement the kernels' lane layouts
allow.  CPU only: the oracle, the planner (host side) and a float64 replay
of the elimination."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import ties
import dense_linear_solvers_amd as tdls


def _sizes(dtype, n, nrhs, monkeypatch):
    out = []
    for t in (4, 16, 64):
        monkeypatch.setenv("TDLS_GROUP_SIZE", str(t))
        rc, _ = tdls.tdls_plan_gesv(tdls.F64 if dtype == "f64" else tdls.F32, tdls.ROW_MAJOR, n,
                                    nrhs, 1)
        if rc == 0:
            out.append(t)
    monkeypatch.delenv("TDLS_GROUP_SIZE")
    return out


@pytest.mark.parametrize("n,dtype,nrhs", ties.SHAPES)
def test_tie_inputs_cover_every_arrangement(n, dtype, nrhs, monkeypatch):
    A = ties.tie_batch(n, dtype)
    _, ipiv, info, gap = oracle.getrf(np.ascontiguousarray(A), n, "row")
    assert (info == 0).all()               # non-singular: the choice shows in piv
    assert (gap == 0).all()                # every system has an exact tie
    sizes = _sizes(dtype, n, nrhs, monkeypatch)
    assert sizes
    for T in sizes:
        R = -(-n // T)
        events, agree = ties.replay_ties(A.astype(np.float64), T, R > 1, ipiv,
                                         is64=dtype == "f64")
        # numpy's argmax takes the first maximum: on the systems whose replay
        # stays exact it agrees with the oracle's pivots
        assert agree.mean() > 0.25, (T, agree.mean())
        c = ties.classify(events)
        assert c["across_lanes"] > 0, (T, c)
        assert c["lower_position_higher_lane"] > 0, (T, c)
        if R > 1:
            assert c["same_lane_two_slots"] > 0, (T, c)
        if dtype == "f64":
            assert c["equal_high_word"] > 0, (T, c)


def test_planted_tie_reaches_its_step_unchanged():
    """Column k of the non-pivot rows reaches step k bit for bit: the oracle's
    pivot at step k is the lower-positioned of the two rows holding +-v, and
    steps 0..k-1 take the planted diagonal rows."""
    rng = np.random.default_rng(3)
    for dtype, npdt in (("f32", np.float32), ("f64", np.float64)):
        for k in (0, 5, 17):
            A = ties.planted_tie(rng, 30, 32, k, npdt).astype(npdt)
            _, ipiv, info, _ = oracle.getrf(np.ascontiguousarray(A), 32, "row")
            assert (info == 0).all()
            v = npdt(1 + 2.0 ** (-40 if dtype == "f64" else -20))
            for s in range(30):
                order = list(range(32))
                for j in range(k):          # positions after steps 0..k-1
                    p = ipiv[s, j]
                    order[j], order[p] = order[p], order[j]
                    assert A[s, order[j], j] == 4.0
                cand = [q for q in range(k, 32) if abs(A[s, order[q], k]) == v]
                assert len(cand) == 2
                assert ipiv[s, k] == min(cand)
