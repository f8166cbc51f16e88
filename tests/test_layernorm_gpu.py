"""LayerNorm forward and backward through the C ABI (layernorm_forward,
layernorm_backward and their bf16 forms) against the fp64 oracle, element
by element, on seeded inputs: the GPT-2 activation shape (8*1024 rows of
768), ragged and tiny shapes, rows kept in registers (C % 4 == 0 and
C <= 2048: 1 to 8 float4 chunks per lane, the last one partly filled) and
rows read twice (longer ones), rows whose length is not a multiple of 4
(scalar loads), rows with a large mean against their spread, constant
rows, and a repeat that must be bitwise equal.

Tolerances, from the arithmetic (fp32 sums of products of O(1) values):
  * fp32 out and dinp: |err| <= 2e-5 + 1e-4 |ref|; mean, rstd: 1e-5 relative;
  * dweight, dbias: sums over N rows of dout * xhat and of dout, added in
    fp32 in chunks of >= 16 rows and then chunk by chunk (a few hundred
    roundings at most, ~1e-5 of the sum of the terms' magnitudes at worst).
    xhat comes from the forward's fp32 mean and rstd, which this test bounds
    by 1e-6 (+1e-5 relative) and 1e-5 relative: a row's xhat is then off by
    up to 1e-6 rstd absolute (the mean's error, which does not shrink with
    xhat) plus 1e-5 |xhat|, times |dout| in dweight:
    |err dweight| <= sum_r |dout| (1e-6 rstd + 1e-5 |xhat|) + 1e-5 sum_r |term| + 1e-4 |ref|,
    |err dbias| <= 1e-5 sum_r |dout| + 1e-4 |ref|;
  * bf16 out and dinp are rounded to bfloat16 (relative 2^-9), so
    2e-2 + 2e-2 |ref|, the same bound as the 16-bit attention outputs;
    fp16 ones to IEEE half (relative 2^-11): 2e-3 + 2e-3 |ref|;
    mean, rstd, dweight and dbias stay fp32 and keep the fp32 bounds.
The oracle sees the same (bf16-rounded, where bf16) input values."""
import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_attn_amd as la
from workloads import randn

pytestmark = pytest.mark.gpu

SHAPES = [(8 * 1024, 768, 0.0), (1, 1, 0.0), (3, 5, 0.0), (17, 64, 0.0), (257, 1000, 3.0),
          (100, 2050, 0.0), (5, 4097, -1.5), (33, 7, 0.0), (2, 8192, 0.0), (64, 2048, 0.5),
          (31, 1536, 0.0), (9, 256, 0.0), (7, 260, 0.0), (12, 1100, 0.0), (10, 1700, 0.0)]


def _inputs(N, C, loc, dtype, seed):
    x = randn((N, C), seed) + loc
    dy = randn((N, C), seed + 1)
    w = 1.0 + 0.5 * randn((C,), seed + 2)
    b = randn((C,), seed + 3)
    if dtype in ("bf16", "f16"):
        t = torch.bfloat16 if dtype == "bf16" else torch.float16
        x, dy = x.to(t), dy.to(t)
    return x, dy, w, b


def _close(got, ref, atol, rtol, what):
    got = got.double().cpu().numpy()
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} beyond bound, max err {err.max():.3g}"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N,C,loc", SHAPES)
def test_layernorm_matches_oracle(N, C, loc, dtype):
    print(f"layernorm {dtype} N={N} C={C} loc={loc}", flush=True)
    x, dy, w, b = _inputs(N, C, loc, dtype, 700 + C)
    ref_out, ref_mean, ref_rstd = oracle.layernorm_forward(x.double().numpy(), w.numpy(), b.numpy())
    ref_dx, ref_dw, ref_db = oracle.layernorm_backward(dy.double().numpy(), x.double().numpy(),
                                                       w.numpy())
    xg, dyg, wg, bg = x.cuda(), dy.cuda(), w.cuda(), b.cuda()
    out, mean, rstd = la.layernorm(xg, wg, bg)
    dx, dw, db = la.layernorm_grad(dyg, xg, wg, mean, rstd)
    torch.cuda.synchronize()
    big = {"bf16": 2e-2, "f16": 2e-3}.get(dtype)
    _close(out, ref_out, big or 2e-5, big or 1e-4, "out")
    _close(mean, ref_mean, 1e-6, 1e-5, "mean")
    _close(rstd, ref_rstd, 0.0, 1e-5, "rstd")
    _close(dx, ref_dx, big or 2e-5, big or 1e-4, "dinp")
    xd, dyd = x.double().numpy(), dy.double().numpy()
    xhat = (xd - ref_mean[:, None]) * ref_rstd[:, None]
    dw_bound = (np.abs(dyd) * (1e-6 * ref_rstd[:, None] + 1e-5 * np.abs(xhat))).sum(axis=0) \
        + 1e-5 * np.abs(dyd * xhat).sum(axis=0)
    _close(dw, ref_dw, dw_bound, 1e-4, "dweight")
    _close(db, ref_db, 1e-5 * np.abs(dyd).sum(axis=0), 1e-4, "dbias")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layernorm_constant_rows(dtype):
    """A constant row has zero variance: out is the bias exactly, the mean is
    the row's value and rstd is 1/sqrt(1e-5); the input gradient is then
    rstd * (dout - mean(dout)) with weight 1 (xhat is 0)."""
    N, C = 6, 768
    x = torch.full((N, C), 2.5)
    x[3] = -7.0
    w, b = torch.ones(C), randn((C,), 91)
    dy = randn((N, C), 92)
    if dtype == "bf16":
        x, dy = x.to(torch.bfloat16), dy.to(torch.bfloat16)
    xg = x.cuda()
    out, mean, rstd = la.layernorm(xg, w.cuda(), b.cuda())
    dx, _, _ = la.layernorm_grad(dy.cuda(), xg, w.cuda(), mean, rstd)
    torch.cuda.synchronize()
    expect_b = b.to(torch.bfloat16).float() if dtype == "bf16" else b
    assert torch.equal(out.float().cpu(), expect_b.expand(N, C))
    assert torch.equal(mean.cpu(), x.float()[:, 0])
    assert torch.allclose(rstd.cpu(), torch.full((N,), 1e-5).rsqrt(), rtol=1e-6, atol=0)
    d = dy.double()
    ref = (d - d.mean(dim=1, keepdim=True)) * (1e-5 ** -0.5)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert torch.allclose(dx.double().cpu(), ref, rtol=tol, atol=tol * 316)


def test_layernorm_backward_is_deterministic():
    N, C = 4096, 768
    x, dy, w, b = _inputs(N, C, 0.0, "f32", 55)
    xg, dyg, wg = x.cuda(), dy.cuda(), w.cuda()
    _, mean, rstd = la.layernorm(xg, wg, b.cuda())
    r1 = la.layernorm_grad(dyg, xg, wg, mean, rstd)
    r2 = la.layernorm_grad(dyg, xg, wg, mean, rstd)
    torch.cuda.synchronize()
    for a, c in zip(r1, r2):
        assert torch.equal(a, c)


def test_layernorm_on_torch_stream():
    """The calls are enqueued on torch's current stream, behind the copy
    that fills their input on that stream."""
    N, C = 4096, 768
    x, dy, w, b = _inputs(N, C, 0.5, "f32", 77)
    ref_out, _, _ = oracle.layernorm_forward(x.double().numpy(), w.numpy(), b.numpy())
    ref_dx, _, _ = oracle.layernorm_backward(dy.double().numpy(), x.double().numpy(), w.numpy())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xg = torch.empty((N, C), device="cuda")
        dyg = torch.empty((N, C), device="cuda")
        xg.copy_(x.pin_memory(), non_blocking=True)
        dyg.copy_(dy.pin_memory(), non_blocking=True)
        out, mean, rstd = la.layernorm(xg, w.cuda(), b.cuda())
        dx, _, _ = la.layernorm_grad(dyg, xg, w.cuda(), mean, rstd)
    s.synchronize()
    _close(out, ref_out, 2e-5, 1e-4, "out")
    _close(dx, ref_dx, 2e-5, 1e-4, "dinp")


def test_layernorm_graph_replays():
    """Forward and backward captured in a HIP graph (the backward's
    workspace already grown by an eager call) give the eager bits on every
    replay, with eager work in between."""
    N, C = 2048, 768
    x, dy, w, b = _inputs(N, C, 0.0, "f32", 78)
    xg, dyg, wg, bg = x.cuda(), dy.cuda(), w.cuda(), b.cuda()
    out, mean, rstd = torch.empty_like(xg), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
    dx, dw, db = torch.empty_like(xg), torch.empty(C, device="cuda"), torch.empty(C, device="cuda")

    def step():
        la.layernorm_forward(out, mean, rstd, xg, wg, bg, N, C)
        la.layernorm_backward(dx, dw, db, dyg, xg, wg, mean, rstd, N, C)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, mean, rstd, dx, dw, db)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for t in (out, mean, rstd, dx, dw, db):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip((out, mean, rstd, dx, dw, db), eager):
            assert torch.equal(a, e)
