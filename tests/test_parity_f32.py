"""fp32 fused path against the fp64 oracle, element by element
(|gpu - oracle| <= 1e-5 + 1e-4 |oracle|), plus GPU-only invariants."""
import sys

import pytest
import torch

from helpers import assert_atomic_dq_equal, assert_close, gpu_fwd_bwd
from workloads import WORKLOADS, make_inputs, workload_inputs

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


@pytest.mark.parametrize("key", [1, 2])
def test_workload_full_compare(la, oracle_mod, key):
    w = WORKLOADS[key]
    _case(f"f32 workload {key}: {w.label()}")
    qkv, dout = workload_inputs(w)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, w.NH, w.causal)
    ro, rl = oracle_mod.forward(qkv, w.NH, w.causal)
    rd = oracle_mod.backward(qkv, dout, w.NH, w.causal)
    assert_close(out, ro, "f32", "out")
    assert_close(lse, rl, "f32", "lse")
    assert_close(dqkv, rd, "f32", "dqkv")


SHAPES = [
    # B, T, C, NH  (hs = C/NH) -- ragged tails, several tiles, every head size
    (1, 1, 64, 4),
    (2, 2, 64, 1),
    (1, 63, 128, 4),
    (2, 65, 128, 2),
    (1, 100, 96, 3),
    (1, 129, 512, 4),
    (3, 200, 64, 4),
    (1, 333, 256, 2),
    (2, 150, 64, 4),      # hs = 16 over several tiles
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(la, oracle_mod, shape, causal):
    B, T, C, NH = shape
    _case(f"f32 ragged B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv, dout = make_inputs(B, T, C, "f32", seed=100 + T)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, NH, causal)
    ro, rl = oracle_mod.forward(qkv, NH, causal)
    rd = oracle_mod.backward(qkv, dout, NH, causal)
    assert_close(out, ro, "f32", "out")
    assert_close(lse, rl, "f32", "lse")
    assert_close(dqkv, rd, "f32", "dqkv")


TILE_EDGE_SHAPES = [(1, 64, 64, 4), (1, 128, 512, 4), (2, 192, 64, 4), (1, 256, 512, 4),
                    (1, 191, 256, 4), (1, 257, 64, 1)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", TILE_EDGE_SHAPES)
def test_tile_edge_lengths(la, oracle_mod, shape, causal):
    """T at and next to multiples of the 64-row tile (the last tile full,
    one row short, one row over), hs = 16, 64 and 128."""
    B, T, C, NH = shape
    _case(f"f32 tile edge B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv, dout = make_inputs(B, T, C, "f32", seed=300 + T)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, NH, causal)
    ro, rl = oracle_mod.forward(qkv, NH, causal)
    rd = oracle_mod.backward(qkv, dout, NH, causal)
    assert_close(out, ro, "f32", "out")
    assert_close(lse, rl, "f32", "lse")
    assert_close(dqkv, rd, "f32", "dqkv")


def test_gpt2_layer_all_heads(la, oracle_mod):
    """The benchmark's workload (B8 T1024 C768 NH12, causal, fp32) in the
    benchmark's launch configuration; every element of every head is
    compared with the oracle."""
    w = WORKLOADS[3]
    _case(f"f32 workload 3, every head: {w.label()}")
    qkv, dout = workload_inputs(w)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, w.NH, w.causal)
    ro, rl = oracle_mod.forward(qkv, w.NH, True)
    rd = oracle_mod.backward(qkv, dout, w.NH, True)
    assert_close(out, ro, "f32", "out")
    assert_close(lse, rl, "f32", "lse")
    assert_close(dqkv, rd, "f32", "dqkv")


def _recompute_backward(la, qkv, dout, out, lse, NH, causal):
    """dqkv from the atomic-free stages (dQ kernel that recomputes S and dP,
    then dK/dV): bitwise reproducible."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    D = torch.empty((B, NH, T), device="cuda")
    g = torch.empty_like(qkv)
    la.attn_backward_dq(g, D, dout, qkv, out, lse, B, T, C, NH, int(causal))
    la.attn_backward_dkdv(g, dout, qkv, lse, D, B, T, C, NH, int(causal))
    return g


def test_deterministic(la):
    """Two runs on the same inputs: out, lse, dk and dv bitwise identical,
    dq equal up to the order of its atomic sums; the recompute stages
    (no atomics) bitwise identical."""
    qkv, dout = make_inputs(2, 300, 256, "f32", seed=5)
    a = gpu_fwd_bwd(la, qkv, dout, 4, True)
    b = gpu_fwd_bwd(la, qkv, dout, 4, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert_atomic_dq_equal(a[2], b[2], 256)
    q, d = qkv.cuda(), dout.cuda()
    out, lse = la.forward(q, 4, True)
    r1 = _recompute_backward(la, q, d, out, lse, 4, True)
    r2 = _recompute_backward(la, q, d, out, lse, 4, True)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)


def test_causality(la):
    """Changing k and v at positions >= t0 leaves out, lse and dq of rows
    < t0 unchanged (masked probabilities are exactly 0): bitwise for out,
    lse and the recompute stages' dq, up to the order of its atomic sums for
    attn_backward's dq."""
    B, T, C, NH = 2, 250, 256, 4
    t0 = 97
    qkv, dout = make_inputs(B, T, C, "f32", seed=6)
    o1, l1, d1 = gpu_fwd_bwd(la, qkv, dout, NH, True)
    qkv2 = qkv.clone()
    qkv2[:, t0:, C:] = 1000.0 * torch.randn_like(qkv2[:, t0:, C:])
    o2, l2, d2 = gpu_fwd_bwd(la, qkv2, dout, NH, True)
    assert torch.equal(o1[:, :t0], o2[:, :t0])
    assert torch.equal(l1[:, :, :t0], l2[:, :, :t0])
    a, b = d1[:, :t0, :C], d2[:, :t0, :C]
    assert (a - b).abs().max().item() <= 1e-5 * a.abs().max().item()
    r = []
    for q in (qkv, qkv2):
        qg, dg = q.cuda(), dout.cuda()
        out, lse = la.forward(qg, NH, True)
        r.append(_recompute_backward(la, qg, dg, out, lse, NH, True).cpu())
    assert torch.equal(r[0][:, :t0, :C], r[1][:, :t0, :C])


def test_first_row_and_single_token_exact(la):
    """Causal row 0 sees only key 0, so out_0 = v_0 exactly; with T = 1
    out = v exactly."""
    B, T, C, NH = 2, 130, 128, 2
    qkv, dout = make_inputs(B, T, C, "f32", seed=7)
    out, _, _ = gpu_fwd_bwd(la, qkv, dout, NH, True)
    assert torch.equal(out[:, 0], qkv[:, 0, 2 * C:])
    qkv1, dout1 = make_inputs(3, 1, C, "f32", seed=8)
    for causal in (True, False):
        out1, _, _ = gpu_fwd_bwd(la, qkv1, dout1, NH, causal)
        assert torch.equal(out1, qkv1[:, :, 2 * C:])


def test_outputs_fully_overwritten(la, oracle_mod):
    """Outputs are written with '=': NaN-filled output buffers come back
    fully defined."""
    B, T, C, NH = 1, 70, 64, 4
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=9)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out = torch.full((B, T, C), float("nan"), device="cuda")
    lse = torch.full((B, NH, T), float("nan"), device="cuda")
    la.attn_forward(out, lse, qkv, B, T, C, NH, 1)
    dqkv = torch.full((B, T, 3 * C), float("nan"), device="cuda")
    la.attn_backward(dqkv, dout, qkv, out, lse, B, T, C, NH, 1)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.forward(qkv_c, NH, True)
    assert_close(out, ro, "f32", "out")
    assert_close(dqkv, oracle_mod.backward(qkv_c, dout_c, NH, True), "f32", "dqkv")


def test_respects_torch_stream(la, oracle_mod):
    """Work is enqueued on torch's current stream."""
    B, T, C, NH = 2, 128, 128, 2
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=10)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qkv = qkv_c.to("cuda", non_blocking=False)
        out, lse = la.forward(qkv, NH, True)
    s.synchronize()
    ro, _ = oracle_mod.forward(qkv_c, NH, True)
    assert_close(out, ro, "f32", "out")


def test_stages_equal_fused_backward(la):
    """attn_backward (fp32) is the pre-pass (D, dq cleared) then the kernel
    that forms dK, dV and adds dQ: the two stage calls give its dk and dv
    bits and its dq up to the order of the atomic sums.  The dK/dV part of
    that kernel is the plain dK/dV kernel's arithmetic: from the same D it
    gives the same dk and dv bits.  The recompute stages (dQ kernel forming
    its own D, then dK/dV) and the dS block store order (pre-pass D, dK/dV
    writing dS, dQ from dS) agree up to fp32 summation order."""
    B, T, C, NH = 2, 300, 256, 4
    _case(f"f32 stages B{B} T{T} C{C} NH{NH}")
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=33)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, lse = la.forward(qkv, NH, True)
    ref = la.backward(dout, qkv, out, lse, NH, True)
    nan = float("nan")
    D1 = torch.full((B, NH, T), nan, device="cuda")
    g1 = torch.full_like(qkv, nan)
    la.attn_backward_prepare(g1, D1, dout, out, B, T, C, NH)
    la.attn_backward_dkdvdq(g1, dout, qkv, lse, D1, B, T, C, NH, 1)
    D2 = torch.full((B, NH, T), nan, device="cuda")
    g2 = torch.full_like(qkv, nan)
    la.attn_backward_dq(g2, D2, dout, qkv, out, lse, B, T, C, NH, 1)
    la.attn_backward_dkdv(g2, dout, qkv, lse, D2, B, T, C, NH, 1)
    D = torch.full((B, NH, T), nan, device="cuda")
    dS = torch.full((la.attn_backward_ds_bytes(B, T, C, NH, 1) // 4,), nan, device="cuda")
    g = torch.full_like(qkv, nan)
    la.attn_backward_preprocess(D, dout, out, B, T, C, NH)
    la.attn_backward_dkdv_ds(g, dS, dout, qkv, lse, D, B, T, C, NH, 1)
    la.attn_backward_dq_ds(g, dS, qkv, B, T, C, NH, 1)
    g3 = torch.full_like(qkv, nan)
    la.attn_backward_dkdv(g3, dout, qkv, lse, D, B, T, C, NH, 1)
    torch.cuda.synchronize()
    assert_atomic_dq_equal(g1, ref, C, "prepare + dkdvdq")
    assert torch.equal(D1, D)                      # the same pre-pass kernel
    assert torch.equal(g3[:, :, C:], ref[:, :, C:])
    assert torch.equal(g3[:, :, C:], g[:, :, C:])
    torch.testing.assert_close(D2, D, rtol=1e-5, atol=1e-5)
    torch.testing.assert_close(g2, ref, rtol=1e-5, atol=1e-5)
    torch.testing.assert_close(g, ref, rtol=1e-5, atol=1e-5)


def test_prepare_clears_dq_only(la):
    """attn_backward_prepare writes D (the same bits attn_backward_preprocess
    writes) and zeros over the dq third of dqkv, and leaves the dk and dv
    thirds as they were."""
    B, T, C, NH = 2, 97, 128, 2
    _case(f"f32 prepare B{B} T{T} C{C} NH{NH}")
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=35)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, _ = la.forward(qkv, NH, True)
    g = torch.full_like(qkv, float("nan"))
    D = torch.full((B, NH, T), float("nan"), device="cuda")
    D2 = torch.full((B, NH, T), float("nan"), device="cuda")
    la.attn_backward_prepare(g, D, dout, out, B, T, C, NH)
    la.attn_backward_preprocess(D2, dout, out, B, T, C, NH)
    torch.cuda.synchronize()
    assert torch.equal(D, D2)
    assert torch.equal(g[:, :, :C], torch.zeros_like(g[:, :, :C]))
    assert torch.isnan(g[:, :, C:]).all()


def test_dkdvdq_adds_into_dq(la, oracle_mod):
    """attn_backward_dkdvdq adds its dq into the dq third and overwrites dk
    and dv: run twice after one attn_backward_prepare, dq is twice the
    gradient and dk, dv are unchanged; on a ragged non-causal shape whose
    last key tile runs past T."""
    B, T, C, NH = 2, 161, 256, 4
    _case(f"f32 dkdvdq accumulation B{B} T{T} C{C} NH{NH}")
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=34)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, lse = la.forward(qkv, NH, False)
    D = torch.empty((B, NH, T), device="cuda")
    g = torch.full_like(qkv, float("nan"))
    la.attn_backward_prepare(g, D, dout, out, B, T, C, NH)
    la.attn_backward_dkdvdq(g, dout, qkv, lse, D, B, T, C, NH, 0)
    once = g.clone()
    la.attn_backward_dkdvdq(g, dout, qkv, lse, D, B, T, C, NH, 0)
    torch.cuda.synchronize()
    assert_close(once, oracle_mod.backward(qkv_c, dout_c, NH, False), "f32", "dqkv")
    assert torch.equal(g[:, :, C:], once[:, :, C:])
    torch.testing.assert_close(g[:, :, :C], 2 * once[:, :, :C], rtol=1e-5, atol=1e-5)


RECOMPUTE_SHAPES = [(1, 1, 64, 4), (2, 65, 128, 2), (1, 100, 96, 3), (1, 129, 512, 4),
                    (1, 333, 256, 2), (2, 150, 64, 4)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", RECOMPUTE_SHAPES)
def test_recompute_stages_ragged(la, oracle_mod, shape, causal):
    """The two stage calls the fused fp32 backward runs (the dQ kernel that
    recomputes S and dP and writes D, then dK/dV), against the oracle."""
    B, T, C, NH = shape
    _case(f"f32 recompute stages B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=200 + T)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    c = int(causal)
    out, lse = la.forward(qkv, NH, causal)
    D = torch.empty((B, NH, T), device="cuda")
    g = torch.full_like(qkv, float("nan"))
    la.attn_backward_dq(g, D, dout, qkv, out, lse, B, T, C, NH, c)
    la.attn_backward_dkdv(g, dout, qkv, lse, D, B, T, C, NH, c)
    torch.cuda.synchronize()
    assert_close(g, oracle_mod.backward(qkv_c, dout_c, NH, causal), "f32", "dqkv")


@pytest.mark.parametrize("causal", [True, False])
def test_ds_stages_ragged(la, oracle_mod, causal):
    """The dS block store stages called directly, on a ragged shape with a
    tail tile (keys >= T in the last tile must carry dS = 0)."""
    B, T, C, NH = 2, 161, 256, 4
    _case(f"f32 dS stages B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=61)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    c = int(causal)
    out, lse = la.forward(qkv, NH, causal)
    D = torch.empty((B, NH, T), device="cuda")
    dS = torch.full((la.attn_backward_ds_bytes(B, T, C, NH, c) // 4,), float("nan"), device="cuda")
    g = torch.full_like(qkv, float("nan"))
    la.attn_backward_preprocess(D, dout, out, B, T, C, NH)
    la.attn_backward_dkdv_ds(g, dS, dout, qkv, lse, D, B, T, C, NH, c)
    la.attn_backward_dq_ds(g, dS, qkv, B, T, C, NH, c)
    torch.cuda.synchronize()
    assert torch.isfinite(dS).all()
    assert_close(g, oracle_mod.backward(qkv_c, dout_c, NH, causal), "f32", "dqkv")
