"""Reader for the hand-worked fixtures under tests/golden/."""
from __future__ import annotations

import glob
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _parse_matrix(text: str) -> np.ndarray:
    rows = [r.split() for r in text.split(";")]
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float64)


def load(path: str) -> dict:
    out = {"name": os.path.basename(path)}
    with open(path, encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            key = key.strip()
            val = val.strip()
            if key in ("A", "L", "U"):
                out[key] = _parse_matrix(val)
            elif key in ("b", "x"):
                out[key] = np.array([float(v) for v in val.split()], dtype=np.float64)
            elif key in ("piv", "ipiv"):
                out[key] = np.array([int(v) for v in val.split()], dtype=np.int32)
            elif key in ("info", "getrf_info"):
                out[key] = int(val)
    return out


def all_examples() -> list:
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "e*.txt")))]


def embed_identity(ex: dict, n: int) -> dict:
    """blockdiag(E, I): the identity rows never win a pivot search against a
    row of E and never change the status, so piv extends with k -> k."""
    m = ex["A"].shape[0]
    A = np.eye(n)
    A[:m, :m] = ex["A"]
    b = np.zeros(n)
    b[:m] = ex["b"]
    out = dict(ex)
    out["A"] = A
    out["b"] = b
    failed = ex["info"] != 0
    out["x"] = np.zeros(n) if failed else np.concatenate([ex["x"], np.zeros(n - m)])
    out["piv"] = (np.full(n, -1, np.int32) if failed
                  else np.concatenate([ex["piv"], np.arange(m, n, dtype=np.int32)]))
    out["ipiv"] = np.concatenate([ex["ipiv"], np.arange(m, n, dtype=np.int32)])
    out.pop("L", None)
    out.pop("U", None)
    return out
