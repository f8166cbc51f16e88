"""The fp8 forward's tolerances against a model of its rounding (CPU,
oracle only).

rounding_model applies, to the oracle's definition, the roundings the fp8
forward is documented to apply: P = exp(s - max) rounded to E4M3, the
normaliser summed over the rounded P, out rounded to bf16.  On heads of the
GPT-2, ViT and long-context workloads (E4M3 inputs) it passes the checks the
GPU parity tests run (helpers: TOL["fp8"], ROW_TOL["fp8"], LSE_ATOL_FP8),
and results with a zeroed row block or a shifted lse fail them.
rounding_model is test infrastructure, not an implementation of the path."""
import numpy as np
import pytest
import torch

from helpers import LSE_ATOL_FP8, assert_close_scaled, row_scaled_violations
from workloads import WORKLOADS, workload_inputs


def _e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).double().numpy()


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).double().numpy()


def rounding_model(q, k, v, causal):
    """(out (T, hs), lse (T,)) of one head with the fp8 forward's roundings."""
    T, hs = q.shape
    s = (q @ k.T) / np.sqrt(hs)
    if causal:
        s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    m = s.max(1, keepdims=True)
    P = _e4m3(np.exp(s - m))
    lsum = P.sum(1, keepdims=True)
    return _bf16(P @ v / lsum), (m + np.log(lsum))[:, 0]


def _head(oracle_mod, key, b, h):
    w = WORKLOADS[key]
    qkv, _ = workload_inputs(w, "fp8")
    qs = oracle_mod.head_slice(qkv.double().numpy(), b, h, w.NH, packed=True)
    out, lse = oracle_mod.forward(qs, 1, w.causal)
    hs = w.hs
    mo, ml = rounding_model(qs[0, :, :hs], qs[0, :, hs:2 * hs], qs[0, :, 2 * hs:], w.causal)
    return w, out, lse, mo[None], ml[None, None]


CASES = [(3, 0, 0), (3, 7, 11), (4, 64, 5), (5, 0, 3)]


@pytest.mark.parametrize("key,b,h", CASES)
def test_rounding_model_passes_and_broken_results_fail(oracle_mod, key, b, h):
    w, out, lse, mo, ml = _head(oracle_mod, key, b, h)
    assert_close_scaled(mo, out, "fp8", "model out", 1, "rows", w.causal)
    assert np.abs(ml - lse).max() <= LSE_ATOL_FP8
    bad = mo.copy()
    bad[:, -64:] = 0.0                       # the last 64 rows' out zeroed
    ne, nn, _ = row_scaled_violations(bad, out, "fp8", 1, "rows", w.causal)
    assert nn >= 60, (ne, nn)
    assert np.abs((ml + 0.1) - lse).max() > LSE_ATOL_FP8


def test_tolerance_tracks_the_rounding():
    """A coarser rounding of P (2 mantissa bits instead of 3) is caught
    row-wise on the GPT-2 layer's first head: the bounds are not so loose
    that twice the E4M3 error passes."""
    import oracle
    w = WORKLOADS[3]
    qkv, _ = workload_inputs(w, "fp8")
    qs = oracle.head_slice(qkv.double().numpy(), 0, 0, w.NH, packed=True)
    out, _ = oracle.forward(qs, 1, w.causal)
    hs = w.hs
    q, k, v = qs[0, :, :hs], qs[0, :, hs:2 * hs], qs[0, :, 2 * hs:]
    s = (q @ k.T) / np.sqrt(hs)
    s = np.where(np.tril(np.ones(s.shape, bool)), s, -np.inf)
    P = np.exp(s - s.max(1, keepdims=True))
    e = np.floor(np.log2(np.maximum(P, 1e-300)))
    step = 2.0 ** (e - 2)                    # 2 mantissa bits
    Pc = np.where(P > 0, np.round(P / step) * step, 0.0)
    # a systematic, not random, error: every weight below the row max rounded
    # down by one coarse step
    Pc = np.where((P > 0) & (P < 1.0), np.maximum(Pc - step, 0.0), Pc)
    bad = (Pc @ v / Pc.sum(1, keepdims=True))[None]
    ne, nn, _ = row_scaled_violations(bad, out, "fp8", 1, "rows", True)
    assert ne + nn > 0
