"""Interleaved batch storage for the tests (data movement only).

Element e of system s of a batch of systems with E elements each, stored
with W systems interleaved, lives at (s // W) * W * E + (s % W) + e * W
(the single strided form of the TDLS page, section Residency: W = 1 is an
array of structures, W = batch a structure of arrays).  As a tensor this
is [blocks, *per_system_shape, W].
"""
from __future__ import annotations

import numpy as np


def to_interleaved(X: np.ndarray, W: int, fill=0) -> np.ndarray:
    """[batch, *shape] -> [blocks, *shape, W]; slots past the batch hold
    ``fill``."""
    X = np.asarray(X)
    batch = X.shape[0]
    blocks = -(-batch // W)
    pad = np.full((blocks * W,) + X.shape[1:], fill, dtype=X.dtype)
    pad[:batch] = X
    pad = pad.reshape((blocks, W) + X.shape[1:])
    axes = (0,) + tuple(range(2, pad.ndim)) + (1,)
    return np.ascontiguousarray(pad.transpose(axes))


def from_interleaved(Y: np.ndarray, batch: int) -> np.ndarray:
    """[blocks, *shape, W] -> [batch, *shape]."""
    Y = np.asarray(Y)
    nd = Y.ndim
    axes = (0, nd - 1) + tuple(range(1, nd - 1))
    X = Y.transpose(axes).reshape((-1,) + Y.shape[1:-1])
    return np.ascontiguousarray(X[:batch])


def padding_of(Y: np.ndarray, batch: int) -> np.ndarray:
    """The slots of [blocks, *shape, W] past the batch, flattened."""
    W = Y.shape[-1]
    blocks = Y.shape[0]
    tail = blocks * W - batch
    if tail == 0:
        return np.zeros(0, Y.dtype)
    return np.ascontiguousarray(Y[-1, ..., W - tail:]).reshape(-1)
