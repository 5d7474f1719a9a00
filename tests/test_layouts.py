"""The interleaved-storage helpers of the tests against the element
formula of the C interface (host only)."""
from __future__ import annotations

import numpy as np
import pytest

import layouts


@pytest.mark.parametrize("W", [1, 2, 3, 5, 11])
def test_element_formula(W):
    rng = np.random.default_rng(W)
    batch, shape = 11, (3, 4)
    E = 12
    X = rng.standard_normal((batch,) + shape)
    Y = layouts.to_interleaved(X, W, fill=np.nan)
    flat = Y.reshape(-1)
    for s in range(batch):
        for e in range(E):
            assert flat[(s // W) * W * E + (s % W) + e * W] == X[s].reshape(-1)[e]
    np.testing.assert_array_equal(layouts.from_interleaved(Y, batch), X)
    pad = layouts.padding_of(Y, batch)
    assert pad.size == (-(-batch // W) * W - batch) * E and np.isnan(pad).all()


def test_structure_of_arrays_and_array_of_structures():
    X = np.arange(5 * 6).reshape(5, 6)
    np.testing.assert_array_equal(layouts.to_interleaved(X, 5)[0], X.T)   # SoA
    np.testing.assert_array_equal(layouts.to_interleaved(X, 1)[..., 0], X)  # AoS
