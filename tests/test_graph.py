"""The stage entry points under HIP graph capture: a captured forward +
backward, replayed several times with eager work and synchronisations in
between, gives bitwise the results of the same calls made eagerly (the
kernels are deterministic, and none of these calls allocates or clears
memory with a memset; the fp32 dq that attn_backward_dkdvdq sums with
atomics is compared up to the order of those sums)."""
import sys

import pytest
import torch

from helpers import assert_atomic_dq_equal
from workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import transformer_causal_head_attn_amd as m
    m.load()
    return m


def _stages(la, dtype, qkv, dout, out, lse, D, dS, dqkv, B, T, C, NH, c):
    if dtype == "f32":
        return [lambda: la.attn_forward(out, lse, qkv, B, T, C, NH, c),
                lambda: la.attn_backward_dq(dqkv, D, dout, qkv, out, lse, B, T, C, NH, c),
                lambda: la.attn_backward_dkdv(dqkv, dout, qkv, lse, D, B, T, C, NH, c)]
    if dtype == "f32_fused":    # what attn_backward runs
        return [lambda: la.attn_forward(out, lse, qkv, B, T, C, NH, c),
                lambda: la.attn_backward_prepare(dqkv, D, dout, out, B, T, C, NH),
                lambda: la.attn_backward_dkdvdq(dqkv, dout, qkv, lse, D, B, T, C, NH, c)]
    if dtype == "f32_ds":
        return [lambda: la.attn_forward(out, lse, qkv, B, T, C, NH, c),
                lambda: la.attn_backward_preprocess(D, dout, out, B, T, C, NH),
                lambda: la.attn_backward_dkdv_ds(dqkv, dS, dout, qkv, lse, D, B, T, C, NH, c),
                lambda: la.attn_backward_dq_ds(dqkv, dS, qkv, B, T, C, NH, c)]
    if dtype == "bf16_fused":   # T <= 256: the one-workgroup-per-head backward
        return [lambda: la.attn_forward_bf16(out, lse, qkv, B, T, C, NH, c),
                lambda: la.attn_backward_bf16(dqkv, dout, qkv, out, lse, B, T, C, NH, c)]
    return [lambda: la.attn_forward_bf16(out, lse, qkv, B, T, C, NH, c),
            lambda: la.attn_backward_dq_bf16(dqkv, D, dout, qkv, out, lse, B, T, C, NH, c),
            lambda: la.attn_backward_dkdv_bf16(dqkv, dout, qkv, lse, D, B, T, C, NH, c)]


@pytest.mark.parametrize("dtype", ["f32", "f32_fused", "f32_ds", "bf16", "bf16_fused"])
def test_graph_replays_equal_eager(la, dtype):
    B, T, C, NH, c = 2, 150, 256, 4, 1
    print(f"\n[case] graph replay {dtype} B{B} T{T} C{C} NH{NH}", flush=True)
    sys.stdout.flush()
    half = dtype.startswith("bf16")
    qkv_c, dout_c = make_inputs(B, T, C, "bf16" if half else "f32", seed=71)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    tdt = torch.bfloat16 if half else torch.float32
    out = torch.empty((B, T, C), dtype=tdt, device="cuda")
    lse = torch.empty((B, NH, T), device="cuda")
    D = torch.empty((B, NH, T), device="cuda")
    dqkv = torch.empty_like(qkv)
    dS = torch.empty((max(la.attn_backward_ds_bytes(B, T, C, NH, c) // 4, 1),), device="cuda")
    stages = _stages(la, dtype, qkv, dout, out, lse, D, dS, dqkv, B, T, C, NH, c)
    for fn in stages:
        fn()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), dqkv.clone())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in stages:
            fn()
    other = torch.randn_like(qkv_c).cuda()
    for r in range(3):
        for t in (out, lse, dqkv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), dqkv.clone())
        for name, a, b in zip(("out", "lse", "dqkv"), got, ref):
            if dtype == "f32_fused" and name == "dqkv":
                assert_atomic_dq_equal(a, b, C, f"replay {r}")
                continue
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager result"
        # eager work between replays, on the same library state
        o2, l2 = la.forward(other, NH, True)
        la.backward(dout, other, o2, l2, NH, True)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_captured_fused_backward_survives_workspace_growth(la, dtype):
    """A captured fused backward keeps the workspace address it saw; a later
    eager call at a larger shape grows the workspace, which must retire the
    old buffer without freeing it, so the graph's replays still give the
    eager bits.  (T = 300: shorter 16-bit sequences need no workspace.)"""
    B, T, C, NH, c = 2, 300, 256, 4, 1
    print(f"\n[case] workspace growth under a captured {dtype} attn_backward", flush=True)
    torch.cuda.synchronize()
    la.attn_release()           # start from no workspace: the first call sizes it
    sfx = "" if dtype == "f32" else "_bf16"
    bwd = getattr(la, "attn_backward" + sfx)
    qkv_c, dout_c = make_inputs(B, T, C, dtype, seed=72)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, lse = la.forward(qkv, NH, True)
    dqkv = torch.empty_like(qkv)
    bwd(dqkv, dout, qkv, out, lse, B, T, C, NH, c)     # eager: sizes the workspace
    torch.cuda.synchronize()
    ref = dqkv.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bwd(dqkv, dout, qkv, out, lse, B, T, C, NH, c)
    # a shape with 16x the D rows: the workspace must grow
    Bb, Tb = 4, 1200
    qb_c, db_c = make_inputs(Bb, Tb, C, dtype, seed=73)
    qb, db = qb_c.cuda(), db_c.cuda()
    ob, lb = la.forward(qb, NH, True)
    gb = torch.empty_like(qb)
    for r in range(3):
        bwd(gb, db, qb, ob, lb, Bb, Tb, C, NH, c)
        torch.cuda.synchronize()
        dqkv.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if dtype == "f32":    # dq summed with atomics
            assert_atomic_dq_equal(dqkv, ref, C, f"replay {r} after growth")
        else:
            assert torch.equal(dqkv, ref), f"replay {r} after growth differs from the eager result"


def test_fp8_forward_graph_replays(la):
    """attn_forward_fp8 allocates nothing and clears nothing, so it can be
    captured; three replays with eager work in between give the eager bits."""
    B, T, C, NH = 2, 150, 256, 4
    print(f"\n[case] graph replay fp8 forward B{B} T{T} C{C} NH{NH}", flush=True)
    q8 = make_inputs(B, T, C, "fp8", seed=74)[0].cuda()
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, NH, T), device="cuda")
    la.attn_forward_fp8(out, lse, q8, B, T, C, NH, 1)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.attn_forward_fp8(out, lse, q8, B, T, C, NH, 1)
    other = make_inputs(B, 300, C, "fp8", seed=75)[0].cuda()
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"replay {r}: out"
        assert torch.equal(lse, ref[1]), f"replay {r}: lse"
        la.forward_fp8(other, NH, True)
        torch.cuda.synchronize()
