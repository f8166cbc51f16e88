"""Pins of the projection oracle (oracle/projection.py), CPU only: each
catches a plausible mistake (a transposed weight, a dropped bias or
residual, a wrong axis)."""
import json
import os

import numpy as np
import pytest

from oracle.projection import projection

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_computed_case():
    g = json.load(open(os.path.join(HERE, "golden", "projection_2x2.json")))
    assert np.array_equal(projection(g["x"], g["w"], g["bias"]), np.array(g["y_no_residual"]))
    assert np.array_equal(projection(g["x"], g["w"], g["bias"], g["residual"]), np.array(g["y"]))


def test_brute_force_loops():
    rng = np.random.default_rng(3)
    M, K, N = 3, 5, 4
    x, w = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    b, r = rng.standard_normal(N), rng.standard_normal((M, N))
    y = projection(x, w, b, r)
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += x[m][k] * w[n][k]
            assert abs(y[m][n] - (s + b[n] + r[m][n])) < 1e-12


def test_identity_and_zero_weights():
    rng = np.random.default_rng(4)
    x, b, r = rng.standard_normal((6, 8)), rng.standard_normal(8), rng.standard_normal((6, 8))
    assert np.allclose(projection(x, np.eye(8), b), x + b, atol=0, rtol=1e-15)
    assert np.array_equal(projection(x, np.zeros((8, 8)), b, r), np.broadcast_to(b, (6, 8)) + r)


def test_linear_in_x():
    rng = np.random.default_rng(5)
    x1, x2 = rng.standard_normal((4, 16)), rng.standard_normal((4, 16))
    w, b = rng.standard_normal((12, 16)), rng.standard_normal(12)
    lhs = projection(x1 + x2, w, b)
    rhs = projection(x1, w, b) + projection(x2, w, b) - b
    assert np.allclose(lhs, rhs, atol=1e-12)


def test_qkv_thirds_and_heads_are_x_times_their_weights():
    """Packed output [Q | K | V] with Q = X W_Q, W_Q = w[:C].T (D x d_k per
    head): columns h*hs .. of each third are x @ W_part[:, head] + bias."""
    rng = np.random.default_rng(6)
    M, C, NH = 10, 32, 4
    hs = C // NH
    x, w, b = rng.standard_normal((M, C)), rng.standard_normal((3 * C, C)), rng.standard_normal(3 * C)
    y = projection(x, w, b)
    for p in range(3):
        Wp = w[p * C:(p + 1) * C].T            # (D, C): columns = output features
        for h in range(NH):
            cols = slice(p * C + h * hs, p * C + (h + 1) * hs)
            ref = x @ Wp[:, h * hs:(h + 1) * hs] + b[cols]
            assert np.allclose(y[:, cols], ref, atol=1e-12)


def test_shape_errors():
    with pytest.raises(ValueError):
        projection(np.zeros((2, 3)), np.zeros((4, 2)), np.zeros(4))
    with pytest.raises(ValueError):
        projection(np.zeros((2, 3)), np.zeros((4, 3)), np.zeros(3))
