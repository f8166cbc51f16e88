"""Materialised fp32 mode (full (B,NH,T,T) preatt/att/datt/dpreatt) against
the fp64 oracle's materialised outputs, element by element at the fp32
tolerance, plus exact zeros under the mask and agreement with the fused
path."""
import pytest
import torch

from helpers import assert_close
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


def run_mat(la, qkv_c, dout_c, NH, causal):
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    out, pre, att = la.forward_materialized(qkv, NH, causal)
    dqkv, dpre, datt = la.backward_materialized(dout, qkv, att, NH, causal)
    torch.cuda.synchronize()
    return [x.cpu() for x in (out, pre, att, dqkv, dpre, datt)]


def compare_all(oracle_mod, got, qkv, dout, NH, causal):
    out, pre, att, dqkv, dpre, datt = got
    ro, _, rp, ra = oracle_mod.forward(qkv, NH, causal, materialized=True)
    rd, rdp, rda = oracle_mod.backward(qkv, dout, NH, causal, materialized=True)
    assert_close(pre, rp, "f32", "preatt")
    assert_close(att, ra, "f32", "att")
    assert_close(out, ro, "f32", "out")
    assert_close(datt, rda, "f32", "datt")
    assert_close(dpre, rdp, "f32", "dpreatt")
    assert_close(dqkv, rd, "f32", "dqkv")


def test_small_workload(la, oracle_mod):
    w = WORKLOADS[2]
    _case(f"materialised workload 2: {w.label()}")
    qkv, dout = workload_inputs(w)
    got = run_mat(la, qkv, dout, w.NH, w.causal)
    compare_all(oracle_mod, got, qkv, dout, w.NH, w.causal)
    T = w.T
    upper = torch.triu(torch.ones(T, T, dtype=torch.bool), 1)
    assert torch.all(got[2][..., upper] == 0.0)      # att
    assert torch.all(got[4][..., upper] == 0.0)      # dpreatt
    rows = got[2].double().sum(-1)
    assert torch.max(torch.abs(rows - 1.0)) < 1e-5


SHAPES = [(1, 1, 64, 4), (2, 63, 128, 4), (1, 65, 128, 2), (2, 100, 96, 3), (1, 130, 512, 4)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(la, oracle_mod, shape, causal):
    B, T, C, NH = shape
    _case(f"materialised ragged B{B} T{T} C{C} NH{NH} causal={causal}")
    qkv, dout = make_inputs(B, T, C, "f32", seed=500 + T)
    got = run_mat(la, qkv, dout, NH, causal)
    compare_all(oracle_mod, got, qkv, dout, NH, causal)


def test_agrees_with_fused_path(la):
    """Materialised and fused paths give the same out and dqkv."""
    B, T, C, NH = 2, 300, 256, 4
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=77)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    for causal in (True, False):
        out, lse = la.forward(qkv, NH, causal)
        dqkv = la.backward(dout, qkv, out, lse, NH, causal)
        out_m, _, att = la.forward_materialized(qkv, NH, causal)
        dqkv_m, _, _ = la.backward_materialized(dout, qkv, att, NH, causal)
        torch.cuda.synchronize()
        assert_close(out_m, out.cpu().double().numpy(), "f32", "out")
        assert_close(dqkv_m, dqkv.cpu().double().numpy(), "f32", "dqkv")


def test_upper_triangle_of_att_is_ignored(la):
    """In causal mode the backward reads only the lower triangle of att."""
    B, T, C, NH = 1, 150, 128, 2
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=78)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    _, _, att = la.forward_materialized(qkv, NH, True)
    d1, p1, a1 = la.backward_materialized(dout, qkv, att, NH, True)
    att2 = att.clone()
    upper = torch.triu(torch.ones(T, T, dtype=torch.bool, device="cuda"), 1)
    att2[..., upper] = 123.0
    d2, p2, a2 = la.backward_materialized(dout, qkv, att2, NH, True)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2) and torch.equal(p1, p2) and torch.equal(a1, a2)


def test_gpt2_layer_all_heads(la, oracle_mod):
    """The materialised mode at the GPT-2 layer size (402 MB per T x T
    matrix): every element of every head of every matrix is compared, one
    sequence of the batch at a time on the oracle's side (12 heads)."""
    w = WORKLOADS[3]
    _case(f"materialised workload 3, every head: {w.label()}")
    qkv, dout = workload_inputs(w)
    out, pre, att, dqkv, dpre, datt = run_mat(la, qkv, dout, w.NH, w.causal)
    for b in range(w.B):
        qb, db = qkv[b:b + 1], dout[b:b + 1]
        ro, _, rp, ra = oracle_mod.forward(qb, w.NH, True, materialized=True)
        assert_close(pre[b:b + 1], rp, "f32", f"preatt b={b}")
        assert_close(att[b:b + 1], ra, "f32", f"att b={b}")
        assert_close(out[b:b + 1], ro, "f32", f"out b={b}")
        del rp, ra
        rd, rdp, rda = oracle_mod.backward(qb, db, w.NH, True, materialized=True)
        assert_close(datt[b:b + 1], rda, "f32", f"datt b={b}")
        assert_close(dpre[b:b + 1], rdp, "f32", f"dpreatt b={b}")
        assert_close(dqkv[b:b + 1], rd, "f32", f"dqkv b={b}")
