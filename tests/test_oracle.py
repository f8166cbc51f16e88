"""Pins for the fp64 CPU oracle (runs without a GPU).

Each test ties the oracle to something other than itself: values derived by
hand from the pages' definitions, closed forms, invariances the mathematics
fixes, torch's own fp64 attention, and central finite differences of the
oracle's forward for its backward.  Every part of the oracle (out, lse,
preatt, att, dqkv, datt, dpreatt) is covered by at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(B, T, C, seed=0, std=1.0):
    qkv, dout = make_inputs(B, T, C, "f32", seed=seed, dout_std=std)
    return qkv.double().numpy(), dout.double().numpy()


def split_heads(qkv, NH):
    """(B,T,3C) -> q, k, v of shape (B,NH,T,hs) (pure indexing)."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    hs = C // NH
    x = qkv.reshape(B, T, 3, NH, hs)
    return [np.ascontiguousarray(x[:, :, p].transpose(0, 2, 1, 3)) for p in range(3)]


# ---------------------------------------------------------------- golden ----

@pytest.mark.parametrize("case", ["causal", "noncausal"])
def test_golden_two_tokens_two_heads(oracle_mod, case):
    with open(os.path.join(GOLDEN, "two_token_two_head.json")) as f:
        g = json.load(f)
    qkv = np.array(g["qkv"], np.float64)
    dout = np.array(g["dout"], np.float64)
    c = g["cases"][case]
    causal = case == "causal"
    out, lse = oracle_mod.forward(qkv, g["NH"], causal)
    np.testing.assert_allclose(out, np.array(c["out"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-13)
    dqkv = oracle_mod.backward(qkv, dout, g["NH"], causal)
    np.testing.assert_allclose(dqkv, np.array(c["dqkv"]), rtol=0, atol=1e-13)


# ---------------------------------------------------------- self-checks ----

@pytest.mark.parametrize("causal", [True, False])
def test_rows_sum_to_one(oracle_mod, causal):
    qkv, _ = rnd(2, 37, 48, seed=11)
    _, _, _, att = oracle_mod.forward(qkv, 3, causal, materialized=True)
    assert np.max(np.abs(att.sum(-1) - 1.0)) <= 1e-12
    assert np.all(att >= 0)


def test_masked_entries_exactly_zero(oracle_mod):
    qkv, dout = rnd(2, 33, 32, seed=12)
    T = 33
    _, _, pre, att = oracle_mod.forward(qkv, 2, True, materialized=True)
    _, dpre, datt = oracle_mod.backward(qkv, dout, 2, True, materialized=True)
    upper = np.triu(np.ones((T, T), bool), 1)
    assert np.all(att[..., upper] == 0.0)
    assert np.all(dpre[..., upper] == 0.0)
    lower = ~upper
    assert np.all(att[..., lower] > 0.0)
    # preatt and datt are dense (masked entries are filled in too)
    assert np.count_nonzero(pre[..., upper]) == pre[..., upper].size
    assert np.count_nonzero(datt[..., upper]) == datt[..., upper].size


@pytest.mark.parametrize("causal", [True, False])
def test_single_token(oracle_mod, causal):
    """T = 1: the only probability is 1, so out = v, lse = scale*q.k,
    dq = dk = 0 and dv = dout, all exactly."""
    B, C, NH = 3, 24, 4
    hs = C // NH
    qkv, dout = rnd(B, 1, C, seed=13)
    out, lse = oracle_mod.forward(qkv, NH, causal)
    q, k, v = split_heads(qkv, NH)
    assert np.array_equal(out, qkv[:, :, 2 * C:])
    ref_lse = (q * k).sum(-1) / math.sqrt(hs)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-14, atol=1e-14)
    dqkv = oracle_mod.backward(qkv, dout, NH, causal)
    assert np.all(dqkv[:, :, :2 * C] == 0.0)
    assert np.array_equal(dqkv[:, :, 2 * C:], dout)


def test_causal_first_row(oracle_mod):
    """Causal row 0 attends to itself only: out = v_0 and dq_0 = 0 exactly."""
    B, T, C, NH = 2, 19, 32, 2
    qkv, dout = rnd(B, T, C, seed=14)
    out, _ = oracle_mod.forward(qkv, NH, True)
    assert np.array_equal(out[:, 0], qkv[:, 0, 2 * C:])
    dqkv = oracle_mod.backward(qkv, dout, NH, True)
    assert np.all(dqkv[:, 0, :C] == 0.0)


@pytest.mark.parametrize("causal", [True, False])
def test_uniform_attention_closed_form(oracle_mod, causal):
    """q = 0 makes every score 0: causal rows are prefix means of v with
    lse = log(t+1); non-causal rows are the mean of v with lse = log T."""
    B, T, C, NH = 2, 23, 32, 4
    qkv, _ = rnd(B, T, C, seed=15)
    qkv[:, :, :C] = 0.0
    out, lse = oracle_mod.forward(qkv, NH, causal)
    v = qkv[:, :, 2 * C:]
    t = np.arange(1, T + 1, dtype=np.float64)
    if causal:
        ref = np.cumsum(v, axis=1) / t[None, :, None]
        ref_lse = np.broadcast_to(np.log(t), lse.shape)
    else:
        ref = np.broadcast_to(v.mean(axis=1, keepdims=True), out.shape)
        ref_lse = np.full(lse.shape, math.log(T))
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_key_shift_invariance(oracle_mod, causal):
    """k_j <- k_j + c for all j adds scale*q.c to every score of a row:
    out is unchanged and lse shifts by scale*q.c."""
    B, T, C, NH = 2, 21, 48, 3
    hs = C // NH
    qkv, _ = rnd(B, T, C, seed=16)
    out0, lse0 = oracle_mod.forward(qkv, NH, causal)
    c = np.random.default_rng(5).standard_normal(C)
    sh = qkv.copy()
    sh[:, :, C:2 * C] += c
    out1, lse1 = oracle_mod.forward(sh, NH, causal)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-12)
    q = qkv[:, :, :C].reshape(B, T, NH, hs)
    shift = (q * c.reshape(NH, hs)).sum(-1).transpose(0, 2, 1) / math.sqrt(hs)
    np.testing.assert_allclose(lse1 - lse0, shift, rtol=1e-11, atol=1e-11)


def test_causal_equals_noncausal_on_prefix(oracle_mod):
    """Causal row t equals the non-causal result on the first t+1 tokens."""
    B, T, C, NH = 1, 17, 16, 2
    qkv, _ = rnd(B, T, C, seed=17)
    out_c, lse_c = oracle_mod.forward(qkv, NH, True)
    for t in (0, 1, 5, 16):
        out_n, lse_n = oracle_mod.forward(qkv[:, :t + 1], NH, False)
        np.testing.assert_allclose(out_c[:, t], out_n[:, t], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse_c[:, :, t], lse_n[:, :, t], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_materialized_consistency(oracle_mod, causal):
    """att = exp(scale*preatt - lse) on unmasked entries, and preatt is the
    plain q.k product (unscaled) everywhere."""
    B, T, C, NH = 2, 29, 32, 2
    hs = C // NH
    qkv, _ = rnd(B, T, C, seed=18)
    _, lse, pre, att = oracle_mod.forward(qkv, NH, causal, materialized=True)
    q, k, _ = split_heads(qkv, NH)
    np.testing.assert_allclose(pre, q @ k.transpose(0, 1, 3, 2), rtol=1e-13, atol=1e-13)
    mask = np.tril(np.ones((T, T), bool)) if causal else np.ones((T, T), bool)
    rec = np.exp(pre / math.sqrt(hs) - lse[..., None])
    np.testing.assert_allclose(att[..., mask], rec[..., mask], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------ backward pins ----

def test_jacobian_form_equals_closed_form(oracle_mod):
    """dpreatt from the oracle (closed form) equals the softmax Jacobian
    double loop of the page's CPU backward:
    dpreatt[t3] = sum_{t2<=t} scale * att[t2] * (1[t2==t3] - att[t3]) * datt[t2]."""
    B, T, C, NH = 2, 24, 32, 2
    hs = C // NH
    scale = 1.0 / math.sqrt(hs)
    qkv, dout = rnd(B, T, C, seed=19)
    _, _, _, att = oracle_mod.forward(qkv, NH, True, materialized=True)
    _, dpre, datt = oracle_mod.backward(qkv, dout, NH, True, materialized=True)
    ref = np.zeros_like(dpre)
    for b in range(B):
        for h in range(NH):
            for t in range(T):
                a = att[b, h, t]
                d = datt[b, h, t]
                for t2 in range(t + 1):
                    for t3 in range(t + 1):
                        ind = 1.0 if t2 == t3 else 0.0
                        ref[b, h, t, t3] += scale * a[t2] * (ind - a[t3]) * d[t2]
    np.testing.assert_allclose(dpre, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_datt_and_rowsum_identity(oracle_mod, causal):
    """datt = dout_t . v_j for every (t, j); and sum_j att*datt = dout_t . out_t."""
    B, T, C, NH = 2, 26, 32, 4
    qkv, dout = rnd(B, T, C, seed=20)
    out, _, _, att = oracle_mod.forward(qkv, NH, causal, materialized=True)
    _, _, datt = oracle_mod.backward(qkv, dout, NH, causal, materialized=True)
    _, _, v = split_heads(qkv, NH)
    hs = C // NH
    do = dout.reshape(B, T, NH, hs).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(datt, do @ v.transpose(0, 1, 3, 2), rtol=1e-13, atol=1e-13)
    D = (att * datt).sum(-1)
    o = out.reshape(B, T, NH, hs).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(D, (do * o).sum(-1), rtol=1e-12, atol=1e-12)


def _loss(oracle_mod, qkv, dout, NH, causal):
    out, _ = oracle_mod.forward(qkv, NH, causal)
    return float((out * dout).sum())


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences_tiny(oracle_mod, causal):
    """Central differences of L = sum(out * dout) through the oracle's
    forward match every entry of its analytic dqkv (B1 T5 C8 NH2)."""
    B, T, C, NH = 1, 5, 8, 2
    qkv, dout = rnd(B, T, C, seed=21)
    dqkv = oracle_mod.backward(qkv, dout, NH, causal)
    num = np.zeros_like(qkv)
    for idx in np.ndindex(*qkv.shape):
        x = qkv[idx]
        h = 1e-5 * max(1.0, abs(x))
        p = qkv.copy(); p[idx] = x + h
        m = qkv.copy(); m[idx] = x - h
        num[idx] = (_loss(oracle_mod, p, dout, NH, causal) - _loss(oracle_mod, m, dout, NH, causal)) / (2 * h)
    np.testing.assert_allclose(dqkv, num, rtol=1e-6, atol=1e-8)


def test_finite_differences_tiny_workload_sampled(oracle_mod):
    """Same check on 200 sampled entries of the tiny workload shape
    (B1 T64 C64 NH4, causal)."""
    B, T, C, NH = 1, 64, 64, 4
    qkv, dout = rnd(B, T, C, seed=22)
    dqkv = oracle_mod.backward(qkv, dout, NH, True)
    rng = np.random.default_rng(7)
    flat = rng.choice(qkv.size, 200, replace=False)
    for f in flat:
        idx = np.unravel_index(f, qkv.shape)
        x = qkv[idx]
        h = 1e-5 * max(1.0, abs(x))
        p = qkv.copy(); p[idx] = x + h
        m = qkv.copy(); m[idx] = x - h
        num = (_loss(oracle_mod, p, dout, NH, True) - _loss(oracle_mod, m, dout, NH, True)) / (2 * h)
        assert abs(dqkv[idx] - num) <= 1e-8 + 1e-6 * abs(num), (idx, dqkv[idx], num)


# ------------------------------------------- library cross-check (fp64) ----

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 64, 64, 4), (2, 70, 96, 3)])
def test_matches_torch_fp64_attention(oracle_mod, causal, shape):
    """torch's CPU attention in float64 (an independent implementation of
    softmax(QK^T/sqrt(hs))V and of its log-sum-exp) agrees with the oracle,
    and torch autograd through it agrees with the oracle's backward."""
    B, T, C, NH = shape
    hs = C // NH
    qkv, dout = rnd(B, T, C, seed=23)
    out, lse = oracle_mod.forward(qkv, NH, causal)
    dqkv = oracle_mod.backward(qkv, dout, NH, causal)

    x = torch.tensor(qkv, requires_grad=True)
    q, k, v = x.view(B, T, 3, NH, hs).permute(2, 0, 3, 1, 4).unbind(0)
    o, l = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(q, k, v, 0.0, causal)[:2]
    o = o.permute(0, 2, 1, 3).reshape(B, T, C)
    (o * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(out, o.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, l.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dqkv, x.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_head_slice_is_the_head(oracle_mod):
    """The oracle on one head cut out of the packed tensor equals that head
    of the full run (heads are independent)."""
    B, T, C, NH = 2, 40, 64, 4
    hs = C // NH
    qkv, dout = rnd(B, T, C, seed=24)
    out, lse = oracle_mod.forward(qkv, NH, True)
    dqkv = oracle_mod.backward(qkv, dout, NH, True)
    b, h = 1, 2
    qs = oracle_mod.head_slice(qkv, b, h, NH, packed=True)
    ds = oracle_mod.head_slice(dout, b, h, NH, packed=False)
    o1, l1 = oracle_mod.forward(qs, 1, True)
    d1 = oracle_mod.backward(qs, ds, 1, True)
    assert np.array_equal(o1[0], out[b, :, h * hs:(h + 1) * hs])
    assert np.array_equal(l1[0, 0], lse[b, h])
    for p in range(3):
        np.testing.assert_allclose(d1[0, :, p * hs:(p + 1) * hs],
                                   dqkv[b, :, p * C + h * hs:p * C + (h + 1) * hs],
                                   rtol=1e-13, atol=1e-14)


def test_invalid_arguments(oracle_mod):
    qkv, _ = rnd(1, 4, 8)
    with pytest.raises(ValueError):
        oracle_mod.forward(qkv, 3, True)  # C=8 not a multiple of NH=3
    with pytest.raises(ValueError):
        oracle_mod.forward(qkv[:, :, :7], 1, True)


# ------------------------------------------ key-range and query-range block ----
# oracle.forward_block restricts rows and keys; it is pinned to the full
# forward (exact equality where the computation is the same), to the merge
# identity that recombines a split of the key range, and to closed forms.

def merge_parts(parts):
    """Recombine (out, lse) results over disjoint key sets: weights
    exp(lse_p - L) with L = log sum_p exp(lse_p) (plain numpy)."""
    outs = np.stack([o for o, _ in parts])          # (P, B, T, C)
    lses = np.stack([l for _, l in parts])          # (P, B, NH, T)
    L = np.logaddexp.reduce(lses, axis=0)           # (B, NH, T)
    P, B, T, C = outs.shape
    NH = lses.shape[2]
    w = np.exp(lses - L[None])                      # (P, B, NH, T)
    w = np.repeat(w.transpose(0, 1, 3, 2), C // NH, axis=3)   # (P, B, T, C)
    return (w * outs).sum(0), L


@pytest.mark.parametrize("causal", [True, False])
def test_block_full_range_is_forward(oracle_mod, causal):
    qkv, _ = rnd(2, 45, 48, seed=61)
    out, lse = oracle_mod.forward(qkv, 3, causal)
    ob, lb = oracle_mod.forward_block(qkv, 3, causal, 0, 45, 0, 45)
    assert np.array_equal(ob, out) and np.array_equal(lb, lse)


@pytest.mark.parametrize("causal", [True, False])
def test_block_query_range_is_rows_of_forward(oracle_mod, causal):
    qkv, _ = rnd(2, 45, 48, seed=62)
    out, lse = oracle_mod.forward(qkv, 3, causal)
    ob, lb = oracle_mod.forward_block(qkv, 3, causal, 17, 45, 0, 45)
    assert np.array_equal(ob, out[:, 17:]) and np.array_equal(lb, lse[:, :, 17:])
    od, ld = oracle_mod.forward_block(qkv, 3, causal, 44, 45, 0, 45)   # decode row
    assert np.array_equal(od, out[:, 44:]) and np.array_equal(ld, lse[:, :, 44:])


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("cuts", [(20,), (7, 30), (1, 2, 40)])
def test_key_split_merges_to_forward(oracle_mod, causal, cuts):
    T = 45
    qkv, _ = rnd(2, T, 48, seed=63)
    out, lse = oracle_mod.forward(qkv, 3, causal)
    edges = (0,) + cuts + (T,)
    parts = [oracle_mod.forward_block(qkv, 3, causal, 0, T, a, b) for a, b in zip(edges, edges[1:])]
    mo, ml = merge_parts(parts)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)


def test_block_rows_without_keys(oracle_mod):
    """Causal rows before k0 see no key of the range: out 0, lse -inf."""
    qkv, _ = rnd(1, 20, 16, seed=64)
    ob, lb = oracle_mod.forward_block(qkv, 2, True, 0, 20, 12, 20)
    assert np.all(ob[:, :12] == 0.0) and np.all(np.isneginf(lb[:, :, :12]))
    assert np.all(np.isfinite(lb[:, :, 12:]))
    oe, le = oracle_mod.forward_block(qkv, 2, False, 0, 20, 5, 5)      # empty range
    assert np.all(oe == 0.0) and np.all(np.isneginf(le))


def test_block_single_key_closed_form(oracle_mod):
    """One key j: the softmax is 1, so out = v_j and lse = scale q.k_j."""
    qkv, _ = rnd(2, 9, 32, seed=65)
    NH, j = 2, 4
    q, k, v = split_heads(qkv, NH)
    ob, lb = oracle_mod.forward_block(qkv, NH, False, 0, 9, j, j + 1)
    hs = 16
    for h in range(NH):
        np.testing.assert_array_equal(ob[:, :, h * hs:(h + 1) * hs],
                                      np.repeat(v[:, h, j:j + 1], 9, axis=1))
        ref = np.einsum("bti,bi->bt", q[:, h], k[:, h, j]) / math.sqrt(hs)
        np.testing.assert_allclose(lb[:, h], ref, rtol=1e-15, atol=1e-15)


def test_block_invalid_ranges(oracle_mod):
    qkv, _ = rnd(1, 8, 16, seed=66)
    for q0, q1, k0, k1 in [(3, 3, 0, 8), (0, 9, 0, 8), (0, 8, 5, 4), (-1, 8, 0, 8)]:
        with pytest.raises(ValueError):
            oracle_mod.forward_block(qkv, 2, True, q0, q1, k0, k1)
