"""Pins of the oracle's LayerNorm (oracle.c, layernorm part) against things
other than itself: torch's float64 layer_norm and its autograd gradients (a
library routine), a hand-computed row, closed forms (a constant row maps to
the bias; column sums of dout give dbias), invariants of the normalised row
and of the input gradient, and central finite differences of the oracle's
own forward.  The definition followed is that of "llm.c 的中文注解-20240423",
section 1.8 (mean, mean squared deviation, rstd = 1/sqrt(var + 1e-5),
out = (x - mean) * rstd * weight + bias)."""
import math

import numpy as np
import pytest
import torch

import oracle

EPS = 1e-5


def _rand(shape, seed, loc=0.0, scale=1.0):
    g = np.random.default_rng(seed)
    return g.normal(loc, scale, size=shape)


@pytest.mark.parametrize("N,C,loc", [(1, 1, 0.0), (3, 5, 0.0), (17, 64, 0.0), (9, 768, 3.0),
                                     (4, 1000, -2.0)])
def test_forward_matches_torch_f64(N, C, loc):
    x = _rand((N, C), 1 + C, loc)
    w = _rand((C,), 2 + C, 1.0, 0.5)
    b = _rand((C,), 3 + C)
    out, mean, rstd = oracle.layernorm_forward(x, w, b)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (C,), torch.from_numpy(w),
                                         torch.from_numpy(b), eps=EPS).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(x.var(axis=1) + EPS), rtol=1e-12)


@pytest.mark.parametrize("N,C", [(3, 5), (17, 64), (6, 768)])
def test_backward_matches_torch_autograd_f64(N, C):
    x = torch.from_numpy(_rand((N, C), 10 + C)).requires_grad_(True)
    w = torch.from_numpy(_rand((C,), 11 + C, 1.0, 0.5)).requires_grad_(True)
    b = torch.from_numpy(_rand((C,), 12 + C)).requires_grad_(True)
    dy = _rand((N, C), 13 + C)
    y = torch.nn.functional.layer_norm(x, (C,), w, b, eps=EPS)
    y.backward(torch.from_numpy(dy))
    dx, dw, db = oracle.layernorm_backward(dy, x.detach().numpy(), w.detach().numpy())
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dw, w.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(db, b.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_hand_computed_row():
    # x = 1, 2, 3, 4: mean 2.5, variance 1.25, deviations -1.5 .. 1.5
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    out, mean, rstd = oracle.layernorm_forward(x, np.ones(4), np.zeros(4))
    r = 1.0 / math.sqrt(1.25 + EPS)
    assert mean[0] == 2.5
    assert rstd[0] == pytest.approx(r, rel=1e-15)
    np.testing.assert_allclose(out[0], np.array([-1.5, -0.5, 0.5, 1.5]) * r, rtol=1e-15)


def test_constant_row_gives_bias():
    C = 7
    b = _rand((C,), 5)
    out, mean, rstd = oracle.layernorm_forward(np.full((2, C), 3.25), _rand((C,), 6), b)
    assert np.all(out == b)
    assert np.all(mean == 3.25)
    assert rstd[0] == pytest.approx(1.0 / math.sqrt(EPS), rel=1e-15)


def test_normalised_rows_invariants():
    N, C = 11, 300
    x = _rand((N, C), 7, 0.5, 2.0)
    out, _, _ = oracle.layernorm_forward(x, np.ones(C), np.zeros(C))
    var = x.var(axis=1)
    np.testing.assert_allclose(out.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((out ** 2).mean(axis=1), var / (var + EPS), rtol=1e-13)


def test_backward_closed_forms():
    N, C = 13, 40
    x, dy = _rand((N, C), 8), _rand((N, C), 9)
    w = np.ones(C)
    dx, dw, db = oracle.layernorm_backward(dy, x, w)
    # dbias is the column sum of dout; with weight 1 each row of dinp sums to 0,
    # and its product with the normalised row is what eps leaves over:
    # sum(dx * xhat) = rstd * sum(dy * xhat) * eps / (var + eps)
    np.testing.assert_allclose(db, dy.sum(axis=0), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    var = x.var(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + EPS)
    xhat = (x - x.mean(axis=1, keepdims=True)) * rstd
    expect = rstd[:, 0] * (dy * xhat).sum(axis=1) * EPS / (var[:, 0] + EPS)
    np.testing.assert_allclose((dx * xhat).sum(axis=1), expect, rtol=1e-8, atol=1e-14)
    np.testing.assert_allclose(dw, (dy * xhat).sum(axis=0), rtol=1e-12, atol=1e-12)


def test_backward_finite_differences():
    N, C = 3, 6
    x = _rand((N, C), 20)
    w = _rand((C,), 21, 1.0, 0.5)
    b = _rand((C,), 22)
    dy = _rand((N, C), 23)
    dx, dw, db = oracle.layernorm_backward(dy, x, w)

    def loss(xx, ww, bb):
        return float((oracle.layernorm_forward(xx, ww, bb)[0] * dy).sum())

    h = 1e-6
    for r in range(N):
        for c in range(C):
            xp, xm = x.copy(), x.copy()
            xp[r, c] += h
            xm[r, c] -= h
            assert (loss(xp, w, b) - loss(xm, w, b)) / (2 * h) == pytest.approx(dx[r, c], abs=1e-7)
    for c in range(C):
        wp, wm = w.copy(), w.copy()
        wp[c] += h
        wm[c] -= h
        assert (loss(x, wp, b) - loss(x, wm, b)) / (2 * h) == pytest.approx(dw[c], abs=1e-7)
        bp, bm = b.copy(), b.copy()
        bp[c] += h
        bm[c] -= h
        assert (loss(x, w, bp) - loss(x, w, bm)) / (2 * h) == pytest.approx(db[c], abs=1e-7)
