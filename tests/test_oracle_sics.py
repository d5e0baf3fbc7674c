"""Pins of the oracle's SICS block score (CPU only).

The oracle evaluates the definition pair by pair; these tests pin it to the
closed form sum_{i,j} u_i.u_j = |sum_i u_i|^2 and to cases whose value is known
without computing cosines: identical directions, orthogonal rows, a one-row
block, zero rows, per-row rescaling, and opposite pairs."""
import numpy as np
import pytest

import oracle


def test_closed_form_identity():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 50, 3, 16))
    s = oracle.block_sics(x, 8)
    for b in range(2):
        for h in range(3):
            for i in range(7):
                rows = x[b, i * 8:min(50, i * 8 + 8), h]
                u = rows / np.linalg.norm(rows, axis=1, keepdims=True)
                assert s[b, h, i] == pytest.approx(np.sum(u.sum(0) ** 2), rel=1e-12)


def test_known_values():
    e = np.eye(8)
    x = np.zeros((1, 24, 1, 8))
    x[0, 0:8, 0] = e * np.arange(1, 9)[:, None]          # orthogonal rows, any lengths -> 8
    x[0, 8:16, 0] = np.tile([1.0, 2, 0, 0, 0, 0, 0, 0], (8, 1)) * np.arange(1, 9)[:, None]  # parallel -> 64
    x[0, 16, 0] = [3.0, 4, 0, 0, 0, 0, 0, 0]              # one row plus zeros -> 1
    s = oracle.block_sics(x, 8)[0, 0]
    assert s[0] == pytest.approx(8.0) and s[1] == pytest.approx(64.0) and s[2] == pytest.approx(1.0)
    y = np.zeros((1, 2, 1, 4))
    y[0, 0, 0], y[0, 1, 0] = [1.0, 0, 0, 0], [-2.0, 0, 0, 0]   # opposite pair: 1 + 1 - 1 - 1
    assert oracle.block_sics(y, 2)[0, 0, 0] == pytest.approx(0.0, abs=1e-15)


def test_rescaling_rows_and_ragged_tail():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 37, 2, 32))
    c = rng.uniform(0.1, 10.0, size=(1, 37, 2, 1))
    assert np.allclose(oracle.block_sics(x, 16), oracle.block_sics(x * c, 16), rtol=1e-12)
    s = oracle.block_sics(x, 16)
    assert s.shape == (1, 2, 3)
    assert np.all(s[..., 2] <= 5 ** 2 + 1e-9)               # 5-row tail block: at most 25
    assert np.all(s >= -1e-9)                               # a squared norm
