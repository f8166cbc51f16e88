"""fp16 fused path (IEEE half tensors, fp32 accumulation) against the fp64
oracle run on the same fp16-rounded inputs, element by element
(|gpu - oracle| <= 5e-3 + 5e-3 |oracle|)."""
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
    (2, 65, 128, 4),    # hs 32, one row into a second tile
    (1, 200, 256, 4),   # hs 64, ragged
    (2, 150, 256, 2),   # hs 128, ragged
    (1, 260, 512, 4),   # hs 128, five tiles
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(la, oracle_mod, shape, causal):
    B, T, C, NH = shape
    _case(f"f16 ragged B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv, dout = make_inputs(B, T, C, "f16", seed=700 + T)
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, NH, causal)
    ro, rl = oracle_mod.forward(qkv, NH, causal)
    rd = oracle_mod.backward(qkv, dout, NH, causal)
    assert_close(out, ro, "f16", "out")
    assert_close(lse, rl, "f16", "lse")
    assert_close(dqkv, rd, "f16", "dqkv")


@pytest.mark.parametrize("key", [1, 2])
def test_small_workloads_in_f16(la, oracle_mod, key):
    w = WORKLOADS[key]
    _case(f"f16 run of workload {key}: {w.label()}")
    qkv, dout = workload_inputs(w, "f16")
    out, lse, dqkv = gpu_fwd_bwd(la, qkv, dout, w.NH, w.causal)
    ro, rl = oracle_mod.forward(qkv, w.NH, w.causal)
    rd = oracle_mod.backward(qkv, dout, w.NH, w.causal)
    assert_close(out, ro, "f16", "out")
    assert_close(lse, rl, "f16", "lse")
    assert_close(dqkv, rd, "f16", "dqkv")


def test_gpt2_layer_f16_all_heads(la, oracle_mod):
    w = WORKLOADS[3]
    check_workload(la, oracle_mod, w, "f16", None,
                   f"f16 run of workload 3, every head: {w.label()}")


def test_vit_f16_all_heads(la, oracle_mod):
    w = WORKLOADS[4]
    check_workload(la, oracle_mod, w, "f16", None,
                   f"f16 run of workload 4, every head: {w.label()}")


def test_long_context_f16_eight_heads(la, oracle_mod):
    w = WORKLOADS[5]
    check_workload(la, oracle_mod, w, "f16", LONG_CONTEXT_HEADS,
                   f"f16 run of workload 5, 8 of 16 heads: {w.label()}")


def test_deterministic_and_causal(la):
    B, T, C, NH = 2, 300, 256, 2
    t0 = 123
    qkv, dout = make_inputs(B, T, C, "f16", seed=41)
    a = gpu_fwd_bwd(la, qkv, dout, NH, True)
    b = gpu_fwd_bwd(la, qkv, dout, NH, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    qkv2 = qkv.clone()
    qkv2[:, t0:, C:] = (100.0 * torch.randn(qkv2[:, t0:, C:].shape)).to(torch.float16)
    o2, l2, d2 = gpu_fwd_bwd(la, qkv2, dout, NH, True)
    assert torch.equal(a[0][:, :t0], o2[:, :t0])
    assert torch.equal(a[1][:, :, :t0], l2[:, :, :t0])
    assert torch.equal(a[2][:, :t0, :C], d2[:, :t0, :C])


def test_single_token_exact(la):
    qkv, dout = make_inputs(2, 1, 256, "f16", seed=42)
    for causal in (True, False):
        out, _, _ = gpu_fwd_bwd(la, qkv, dout, 4, causal)
        assert torch.equal(out, qkv[:, :, 512:])


def test_stages_equal_fused_backward(la):
    """dq (which writes D) then dkdv equals attn_backward_f16; the standalone
    pre-pass gives the same D."""
    B, T, C, NH = 2, 300, 256, 4
    qkv_c, dout_c = make_inputs(B, T, C, "f16", seed=43)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, lse = la.forward(qkv, NH, True)
    ref = la.backward(dout, qkv, out, lse, NH, True)
    D = torch.full((B, NH, T), float("nan"), device="cuda")
    g = torch.full_like(qkv, float("nan"))
    la.attn_backward_dq_f16(g, D, dout, qkv, out, lse, B, T, C, NH, 1)
    la.attn_backward_dkdv_f16(g, dout, qkv, lse, D, B, T, C, NH, 1)
    D2 = torch.full((B, NH, T), float("nan"), device="cuda")
    la.attn_backward_preprocess_f16(D2, dout, out, B, T, C, NH)
    torch.cuda.synchronize()
    assert torch.equal(g, ref)
    torch.testing.assert_close(D2, D, rtol=1e-5, atol=1e-5)
