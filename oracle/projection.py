"""fp64 CPU oracle of the two projections beside the attention block.

TEST INFRASTRUCTURE ONLY: the test-suite and the benchmark's CPU baseline may
import this module; the HIP library and its binding never do, and the two
share no code.

    projection(x, w, bias, residual=None)[m][n]
        = sum_k x[m][k] * w[n][k] + bias[n] (+ residual[m][n])

With w of shape (N, K) whose rows are the columns of the weight matrices
W_Q, W_K, W_V in Q = X W_Q, K = X W_K, V = X W_V ("Umakini wa kujitegemea,
kerneli za CUDA na FlashAttention", section 1), and N = 3C, this is the
packed (B, T, 3C) qkv; with a residual it is the output projection followed
by residual_forward_kernel's out = inp1 + inp2 ("llm.c 的中文注解-20240423",
section 1.15).  The product is numpy's float64 matmul (a library routine
serving as one step); the bias and the residual are added after it, as the
definition reads.  Pinned by tests/test_oracle_projection.py (brute-force
loops, a hand-computed case, identity and zero weights, linearity, the
per-head slices of Q = X W_Q).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def projection(x, w, bias, residual=None):
    """x (M, K), w (N, K), bias (N,), residual (M, N) or None -> (M, N) float64."""
    x, w, b = _f64(x), _f64(w), _f64(bias)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1] or b.shape != (w.shape[0],):
        raise ValueError(f"shapes x {x.shape}, w {w.shape}, bias {b.shape} do not match")
    y = x @ w.T
    y = y + b[None, :]
    if residual is not None:
        r = _f64(residual)
        if r.shape != y.shape:
            raise ValueError(f"residual {r.shape} does not match {y.shape}")
        y = y + r
    return y
