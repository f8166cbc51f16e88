"""bf16 fused path (bf16 tensors, fp32 accumulation) against the fp64 oracle
run on the same bf16-rounded inputs, element by element
(|gpu - oracle| <= 2e-2 + 2e-2 |oracle|)."""
import pytest
import torch

from helpers import LONG_CONTEXT_HEADS, assert_close, check_workload, gpu_fwd_bwd
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


SHAPES = [
    (1, 1, 64, 4),      # hs 16, single token
    (2, 33, 64, 4),     # hs 16, ragged single tile
    (1, 64, 128, 4),    # hs 32, exactly one tile
    (2, 65, 128, 4),    # hs 32, one row into a second tile
    (1, 200, 256, 4),   # hs 64, ragged
    (2, 150, 256, 2),   # hs 128, ragged
    (1, 260, 512, 4),   # hs 128, five tiles
    (1, 384, 256, 4),   # hs 64, three full 128-row forward tiles (two-kernel backward)
    (1, 383, 512, 4),   # hs 128, one row short of them
    (1, 385, 256, 4),   # hs 64, one row over
    (1, 512, 128, 8),   # hs 16, four full forward tiles
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(la, oracle_mod, shape, causal):
    B, T, C, NH = shape
    _case(f"bf16 ragged B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv, dout = make_inputs(B, T, C, "bf16", seed=300 + T)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, NH, causal)
    ro, rl = oracle_mod.forward(qkv, NH, causal)
    rd = oracle_mod.backward(qkv, dout, NH, causal)
    assert_close(out, ro, "bf16", "out")
    assert_close(lse, rl, "bf16", "lse")
    assert_close(dqkv, rd, "bf16", "dqkv")


@pytest.mark.parametrize("key", [1, 2])
def test_small_workloads_in_bf16(la, oracle_mod, key):
    """The tiny and small workload shapes run through the bf16 path."""
    w = WORKLOADS[key]
    _case(f"bf16 run of workload {key}: {w.label()}")
    qkv, dout = workload_inputs(w, "bf16")
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, w.NH, w.causal)
    ro, rl = oracle_mod.forward(qkv, w.NH, w.causal)
    rd = oracle_mod.backward(qkv, dout, w.NH, w.causal)
    assert_close(out, ro, "bf16", "out")
    assert_close(lse, rl, "bf16", "lse")
    assert_close(dqkv, rd, "bf16", "dqkv")


def test_gpt2_layer_bf16_all_heads(la, oracle_mod):
    w = WORKLOADS[3]
    check_workload(la, oracle_mod, w, "bf16", None,
                   f"bf16 run of workload 3, every head: {w.label()}")


def test_vit_workload_all_heads(la, oracle_mod):
    w = WORKLOADS[4]
    check_workload(la, oracle_mod, w, "bf16", None, f"bf16 workload 4, every head: {w.label()}")


def test_partial_deal_round(la, oracle_mod):
    """B*NH = 80 heads of 8 causal 128-row tiles: 640 unpaired workgroups, so
    the snake deal reverses the second resident round and leaves the third
    partial; every head is checked against the oracle."""
    B, T, C, NH = 8, 1024, 640, 10
    _case(f"bf16 B{B} T{T} C{C} NH{NH} causal, all heads")
    qkv, dout = make_inputs(B, T, C, "bf16", seed=910)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, NH, True)
    ro, rl = oracle_mod.forward(qkv, NH, True)
    rd = oracle_mod.backward(qkv, dout, NH, True)
    assert_close(out, ro, "bf16", "out")
    assert_close(lse, rl, "bf16", "lse")
    assert_close(dqkv, rd, "bf16", "dqkv")


def test_long_context_eight_heads(la, oracle_mod):
    w = WORKLOADS[5]
    check_workload(la, oracle_mod, w, "bf16", LONG_CONTEXT_HEADS,
                   f"bf16 workload 5, 8 of 16 heads: {w.label()}")


def test_deterministic_and_causal(la):
    B, T, C, NH = 2, 300, 256, 2
    t0 = 123
    qkv, dout = make_inputs(B, T, C, "bf16", seed=31)
    a = gpu_fwd_bwd(la, qkv, dout, NH, True)
    b = gpu_fwd_bwd(la, qkv, dout, NH, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    qkv2 = qkv.clone()
    qkv2[:, t0:, C:] = (100.0 * torch.randn(qkv2[:, t0:, C:].shape)).to(torch.bfloat16)
    o2, l2, d2 = gpu_fwd_bwd(la, qkv2, dout, NH, True)
    assert torch.equal(a[0][:, :t0], o2[:, :t0])
    assert torch.equal(a[1][:, :, :t0], l2[:, :, :t0])
    assert torch.equal(a[2][:, :t0, :C], d2[:, :t0, :C])


def test_single_token_exact(la):
    qkv, dout = make_inputs(2, 1, 256, "bf16", seed=32)
    for causal in (True, False):
        out, _, _ = gpu_fwd_bwd(la, qkv, dout, 4, causal)
        assert torch.equal(out, qkv[:, :, 512:])


def test_stages_equal_fused_backward(la):
    """dq (which writes D) then dkdv equals attn_backward_bf16 (T = 300: the
    fused call runs these two kernels); the standalone pre-pass gives the
    same D, and dkdv run from it (before dq) gives the same dk and dv.  (The
    fp32 stages: test_parity_f32.py.)"""
    for dtype in ("bf16",):
        B, T, C, NH = 2, 300, 256, 4
        qkv_c, dout_c = make_inputs(B, T, C, dtype, seed=33)
        qkv, dout = qkv_c.cuda(), dout_c.cuda()
        out, lse = la.forward(qkv, NH, True)
        ref = la.backward(dout, qkv, out, lse, NH, True)
        sfx = "_bf16" if dtype == "bf16" else ""
        D = torch.full((B, NH, T), float("nan"), device="cuda")
        g = torch.full_like(qkv, float("nan"))
        getattr(la, "attn_backward_dq" + sfx)(g, D, dout, qkv, out, lse, B, T, C, NH, 1)
        getattr(la, "attn_backward_dkdv" + sfx)(g, dout, qkv, lse, D, B, T, C, NH, 1)
        D2 = torch.full((B, NH, T), float("nan"), device="cuda")
        getattr(la, "attn_backward_preprocess" + sfx)(D2, dout, out, B, T, C, NH)
        g2 = torch.full_like(qkv, float("nan"))
        getattr(la, "attn_backward_dkdv" + sfx)(g2, dout, qkv, lse, D2, B, T, C, NH, 1)
        torch.cuda.synchronize()
        assert torch.equal(g, ref)
        # the two D's differ only in summation order
        torch.testing.assert_close(D2, D, rtol=1e-5, atol=1e-5)
        tol = 1e-2 if dtype == "bf16" else 1e-5   # bf16: one rounding step
        torch.testing.assert_close(g2[:, :, C:].float(), ref[:, :, C:].float(),
                                   rtol=tol, atol=tol)


SHORT_SHAPES = [
    (2, 196, 768, 12),   # hs 64, ViT length: one workgroup per head
    (3, 200, 256, 16),   # hs 16
    (2, 129, 512, 16),   # hs 32, one row past 128
    (1, 256, 256, 4),    # hs 64, the longest such sequence
    (2, 100, 256, 4),    # hs 64 at T <= 128: the two kernels
    (2, 64, 128, 8),     # hs 16, exactly one query tile
    (2, 256, 128, 8),    # hs 16, every wave's keys below T
    (1, 256, 512, 16),   # hs 32, four full query tiles
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHORT_SHAPES)
def test_short_sequence_backward_paths(la, oracle_mod, shape, causal, dtype):
    """For T <= 256 the fused backward runs one workgroup per head, with the
    head's dS kept in LDS; the stage calls keep the dQ and dK/dV kernels.
    Both are checked against the oracle on the same inputs."""
    B, T, C, NH = shape
    _case(f"{dtype} short-sequence backward B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv_c, dout_c = make_inputs(B, T, C, dtype, seed=1200 + T)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    sfx = "_" + dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    c = int(causal)
    out = torch.empty((B, T, C), dtype=tdt, device="cuda")
    lse = torch.empty((B, NH, T), device="cuda")
    getattr(la, "attn_forward" + sfx)(out, lse, qkv, B, T, C, NH, c)
    fused = torch.full_like(qkv, float("nan"))
    getattr(la, "attn_backward" + sfx)(fused, dout, qkv, out, lse, B, T, C, NH, c)
    D = torch.full((B, NH, T), float("nan"), device="cuda")
    staged = torch.full_like(qkv, float("nan"))
    getattr(la, "attn_backward_dq" + sfx)(staged, D, dout, qkv, out, lse, B, T, C, NH, c)
    getattr(la, "attn_backward_dkdv" + sfx)(staged, dout, qkv, lse, D, B, T, C, NH, c)
    torch.cuda.synchronize()
    rd = oracle_mod.backward(qkv_c, dout_c, NH, causal)
    assert_close(fused.cpu(), rd, dtype, "dqkv (fused)")
    assert_close(staged.cpu(), rd, dtype, "dqkv (stages)")
