"""QKV projection and output projection (+ residual) GEMMs against the fp64
projection oracle, element by element, at the GPT-2 layer's sizes (M = B*T =
8192 rows, C = 768) and on ragged shapes that leave partial tiles in every
dimension."""
import sys

import numpy as np
import pytest
import torch

from helpers import assert_close
from oracle.projection import projection
from workloads import randn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import transformer_causal_head_attn_amd as m
    m.load()
    return m


def _case(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(M, K, N, dtype, seed, residual):
    """x ~ N(0, 1) (a normalised activation), w ~ N(0, 0.02^2) (GPT-2's
    initialisation scale), bias ~ N(0, 0.02^2) fp32, residual ~ N(0, 1)."""
    x = randn((M, K), seed, 1.0, dtype)
    w = randn((N, K), seed + 1, 0.02, dtype)
    b = randn((N,), seed + 2, 0.02, "f32")
    r = randn((M, N), seed + 3, 1.0, dtype) if residual else None
    return x, w, b, r


def _row_norm_check(g, r, frac, what):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    e = np.sqrt(np.sum((g - r) ** 2, axis=1))
    n = np.sqrt(np.sum(r * r, axis=1)) + 1e-12
    bad = e > frac * n
    assert not bad.any(), f"{what}: {int(bad.sum())} rows with relative 2-norm error > {frac}"


def _run(la, M, K, N, dtype, residual, seed):
    x, w, b, r = _inputs(M, K, N, dtype, seed, residual)
    xg, wg, bg = x.cuda(), w.cuda(), b.cuda()
    if residual:
        y = la.out_projection(xg, wg, bg, r.cuda())
    else:
        y = la.qkv_projection(xg, wg, bg)
    torch.cuda.synchronize()
    ref = projection(x, w, b, r)
    y = y.cpu().double().numpy()
    assert_close(y, ref, dtype, "y")
    # bf16: operands exact, fp32 sums, one rounding of the output (2^-9
    # relative) -> rows agree to well under 1% in the 2-norm
    _row_norm_check(y, ref, 1e-6 if dtype == "f32" else 5e-3, "y")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpt2_qkv_projection(la, dtype):
    _case(f"qkv projection {dtype} M8192 K768 N2304")
    _run(la, 8192, 768, 2304, dtype, False, 2100)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpt2_out_projection_with_residual(la, dtype):
    _case(f"out projection + residual {dtype} M8192 K768 N768")
    _run(la, 8192, 768, 768, dtype, True, 2200)


RAGGED = [(1, 8, 4), (7, 40, 12), (129, 72, 132), (300, 200, 260), (257, 1032, 388)]


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", RAGGED)
def test_ragged(la, shape, dtype, residual):
    M, K, N = shape
    _case(f"projection {dtype} M{M} K{K} N{N} residual={residual}")
    _run(la, M, K, N, dtype, residual, 2300 + M)


def test_qkv_projection_feeds_attention(la, oracle_mod):
    """x -> packed qkv (bf16, the projection's output layout) -> attention
    forward, against the oracle's attention of the oracle's projection of the
    same x rounded to bf16 (the rounding the bf16 path applies to qkv)."""
    B, T, C, NH = 2, 200, 256, 4
    _case(f"projection -> attention bf16 B{B} T{T} C{C} NH{NH}")
    x, w, b, _ = _inputs(B * T, C, 3 * C, "bf16", 2400, False)
    qkv = la.qkv_projection(x.cuda(), w.cuda(), b.cuda()).view(B, T, 3 * C)
    out, lse = la.forward(qkv, NH, True)
    torch.cuda.synchronize()
    ref_qkv = projection(x, w, b).reshape(B, T, 3 * C)
    ref_qkv = torch.from_numpy(ref_qkv).float().to(torch.bfloat16)
    assert_close(qkv.cpu(), ref_qkv.double().numpy(), "bf16", "qkv")
    ro, rl = oracle_mod.forward(ref_qkv, NH, True)
    assert_close(out.cpu(), ro, "bf16", "out")
    assert_close(lse.cpu(), rl, "bf16", "lse")


def test_errors(la):
    x = torch.zeros((4, 12), device="cuda")
    w = torch.zeros((8, 12), device="cuda")
    b = torch.zeros((8,), device="cuda")
    y = torch.zeros((4, 8), device="cuda")
    with pytest.raises(la.AttnError):   # K = 12 not a multiple of 8 in bf16
        la.attn_qkv_projection_bf16(y.to(torch.bfloat16), x.to(torch.bfloat16),
                                    w.to(torch.bfloat16), b, 4, 12, 8)
    with pytest.raises(la.AttnError):   # output overlaps an input
        la.attn_out_projection(y, x, w, b, y, 4, 12, 8)
