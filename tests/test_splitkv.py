"""Split-KV forward (16-bit path): each query tile's keys split into chunks
over workgroups, partial (O, lse) merged per row, against the fp64 oracle
element by element (stated bound and the row-scaled checks), and against the
plain forward."""
import sys

import pytest
import torch

from helpers import (LONG_CONTEXT_HEADS, assert_close, assert_close_scaled, head_view)
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


SHAPES = [
    (1, 1, 64, 4),      # hs 16, one token
    (2, 100, 64, 4),    # hs 16, ragged
    (1, 260, 128, 4),   # hs 32
    (2, 333, 256, 4),   # hs 64, ragged
    (1, 515, 512, 4),   # hs 128, ragged
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("chunk", [64, 128, 192, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_against_oracle(la, oracle_mod, shape, causal, chunk, dtype):
    B, T, C, NH = shape
    _case(f"split-KV {dtype} B{B} T{T} C{C} NH{NH} causal={causal} chunk={chunk}")
    qkv_c, _ = make_inputs(B, T, C, dtype, seed=1300 + T)
    out, lse = la.forward_splitkv(qkv_c.cuda(), NH, causal, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.forward(qkv_c, NH, causal)
    assert_close_scaled(out.cpu(), ro, dtype, "out", NH, "rows", causal)
    assert_close(lse.cpu(), rl, dtype, "lse")


def test_two_long_context_heads_auto_chunk(la, oracle_mod):
    """One GPU's share of the long-context workload under an 8-way head
    split: 2 heads of T = 8192 (hs = 128), 128 query tiles for the plain
    grid.  The library's chunk splits them; every element of both heads
    against the oracle."""
    w = WORKLOADS[5]
    qkv, _ = workload_inputs(w)
    C2 = 2 * w.hs
    # heads 0 and 1 of sequence 0, repacked as a 2-head (1, T, 3*C2) tensor
    q2 = torch.cat([qkv[:, :, p * w.C:p * w.C + C2] for p in range(3)], dim=2).contiguous()
    chunk = la.attn_forward_splitkv_chunk(1, w.T, C2, 2, 1)
    _case(f"split-KV bf16 two long-context heads, chunk {chunk}")
    assert 64 <= chunk < w.T
    out, lse = la.forward_splitkv(q2.cuda(), 2, True, 0)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.forward(q2, 2, True)
    assert_close_scaled(out.cpu(), ro, "bf16", "out", 2, "rows", True)
    assert_close(lse.cpu(), rl, "bf16", "lse")


def test_long_context_explicit_chunk_eight_heads(la, oracle_mod):
    w = WORKLOADS[5]
    _case(f"split-KV bf16 {w.label()}, 1024-key chunks, 8 of 16 heads")
    qkv, _ = workload_inputs(w)
    out, lse = la.forward_splitkv(qkv.cuda(), w.NH, True, 1024)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    x = qkv.double().numpy()
    for b, h in LONG_CONTEXT_HEADS:
        qs = oracle_mod.head_slice(x, b, h, w.NH, packed=True)
        ro, rl = oracle_mod.forward(qs, 1, True)
        assert_close_scaled(head_view(out, b, h, w.NH, False), ro, "bf16", f"out head {(b, h)}",
                            1, "rows", True)
        assert_close(lse[b:b + 1, h:h + 1].numpy(), rl, "bf16", f"lse head {(b, h)}")


def test_agrees_with_plain_forward_and_is_deterministic(la):
    B, T, C, NH = 2, 700, 512, 4
    qkv_c, _ = make_inputs(B, T, C, "bf16", seed=1401)
    qkv = qkv_c.cuda()
    o1, l1 = la.forward(qkv, NH, True)
    o2, l2 = la.forward_splitkv(qkv, NH, True, 128)
    o3, l3 = la.forward_splitkv(qkv, NH, True, 128)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    torch.testing.assert_close(o2.float(), o1.float(), rtol=2e-2, atol=2e-2)
    # both normalisers sum P rounded to bf16 (against different running
    # maxima): lse differs by up to about one bf16 rounding step
    torch.testing.assert_close(l2, l1, rtol=0, atol=2 ** -8)


def test_causality_bitwise(la):
    """Keys and values at positions >= t0 changed: out and lse of rows < t0
    bitwise unchanged under the split too."""
    B, T, C, NH, t0 = 1, 600, 256, 2, 259
    qkv_c, _ = make_inputs(B, T, C, "bf16", seed=1402)
    o1, l1 = la.forward_splitkv(qkv_c.cuda(), NH, True, 128)
    qkv2 = qkv_c.clone()
    qkv2[:, t0:, C:] = (50.0 * torch.randn(qkv2[:, t0:, C:].shape)).to(torch.bfloat16)
    o2, l2 = la.forward_splitkv(qkv2.cuda(), NH, True, 128)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :t0], o2[:, :t0])
    assert torch.equal(l1[:, :, :t0], l2[:, :, :t0])


def test_no_split_leaves_work_untouched(la, oracle_mod):
    """A chunk covering every key runs the plain forward: same bits as
    attn_forward_bf16, and the work buffer is not written."""
    B, T, C, NH = 2, 200, 256, 4
    qkv_c, _ = make_inputs(B, T, C, "bf16", seed=1403)
    qkv = qkv_c.cuda()
    assert la.attn_forward_splitkv_bytes(B, T, C, NH, 1, 256) == 0
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, NH, T), device="cuda")
    work = torch.full((64,), 7.0, device="cuda")
    la.attn_forward_splitkv_bf16(out, lse, qkv, work, B, T, C, NH, 1, 256)
    o1, l1 = la.forward(qkv, NH, True)
    torch.cuda.synchronize()
    assert torch.equal(out, o1) and torch.equal(lse, l1)
    assert torch.all(work == 7.0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("chunk", [64, 192, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_backward_ragged_against_oracle(la, oracle_mod, shape, causal, chunk, dtype):
    B, T, C, NH = shape
    _case(f"split backward {dtype} B{B} T{T} C{C} NH{NH} causal={causal} chunk={chunk}")
    qkv_c, dout_c = make_inputs(B, T, C, dtype, seed=1500 + T)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, lse = la.forward(qkv, NH, causal)
    dqkv = la.backward_splitkv(dout, qkv, out, lse, NH, causal, chunk)
    torch.cuda.synchronize()
    rd = oracle_mod.backward(qkv_c, dout_c, NH, causal)
    assert_close_scaled(dqkv.cpu(), rd, dtype, "dqkv", NH, "packed", causal)


def test_backward_two_long_context_heads(la, oracle_mod):
    """The split backward on one GPU's share of the long-context workload
    (2 heads of T = 8192), the library's chunk; every element of both heads."""
    w = WORKLOADS[5]
    qkv, dout = workload_inputs(w)
    C2 = 2 * w.hs
    q2 = torch.cat([qkv[:, :, p * w.C:p * w.C + C2] for p in range(3)], dim=2).contiguous()
    d2 = dout[:, :, :C2].contiguous()
    _case("split backward bf16 two long-context heads, library chunk")
    qg, dg = q2.cuda(), d2.cuda()
    out, lse = la.forward_splitkv(qg, 2, True, 0)
    dqkv = la.backward_splitkv(dg, qg, out, lse, 2, True, 0)
    torch.cuda.synchronize()
    rd = oracle_mod.backward(q2, d2, 2, True)
    assert_close_scaled(dqkv.cpu(), rd, "bf16", "dqkv", 2, "packed", True)


def test_backward_split_agrees_with_plain_and_is_deterministic(la):
    B, T, C, NH = 2, 700, 512, 4
    qkv_c, dout_c = make_inputs(B, T, C, "bf16", seed=1501)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, lse = la.forward(qkv, NH, True)
    ref = la.backward(dout, qkv, out, lse, NH, True)
    g1 = la.backward_splitkv(dout, qkv, out, lse, NH, True, 128)
    g2 = la.backward_splitkv(dout, qkv, out, lse, NH, True, 128)
    g3 = la.backward_splitkv(dout, qkv, out, lse, NH, True, 1024)   # no split
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    assert torch.equal(g3, ref)
    torch.testing.assert_close(g1.float(), ref.float(), rtol=2e-2, atol=2e-2)
