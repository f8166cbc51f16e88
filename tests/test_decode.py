"""Decode (the last query row against every key, split over key ranges) and
the (O, lse) merge of partial results, against the fp64 oracle's
forward_block on the same seeded inputs."""
import numpy as np
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


def _decode_ref(oracle_mod, qkv, NH):
    T = qkv.shape[1]
    out, lse = oracle_mod.forward_block(qkv, NH, True, T - 1, T, 0, T)
    return out[:, 0], lse[:, :, 0]


DECODE_SHAPES = [
    (1, 1, 64, 4),       # hs 16, a single key
    (2, 5, 128, 4),      # hs 32
    (2, 127, 256, 4),    # hs 64, one range short of 128
    (1, 128, 256, 4),    # exactly one 128-key range
    (3, 129, 256, 4),    # one key into a second range
    (2, 300, 512, 4),    # hs 128, ragged
    (1, 777, 64, 4),     # hs 16, many ranges
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_decode_shapes(la, oracle_mod, shape, dtype):
    B, T, C, NH = shape
    _case(f"decode {dtype} B{B} T{T} C{C} NH{NH}")
    qkv, _ = make_inputs(B, T, C, dtype, seed=500 + T)
    out, lse = la.decode(qkv.cuda(), NH)
    torch.cuda.synchronize()
    ro, rl = _decode_ref(oracle_mod, qkv, NH)
    assert_close(out.cpu(), ro, dtype, "decode out")
    assert_close(lse.cpu(), rl, dtype, "decode lse")


@pytest.mark.parametrize("key,dtype", [(3, "f32"), (3, "bf16"), (5, "bf16"), (4, "bf16"), (5, "f16")])
def test_decode_workload_caches(la, oracle_mod, key, dtype):
    """Decode over the full-size inputs of the GPT-2 layer, long-context and
    ViT workloads (every (b, h) row checked: one row per head is cheap)."""
    w = WORKLOADS[key]
    _case(f"decode {dtype} over workload {key}: {w.label()}")
    qkv, _ = workload_inputs(w, dtype)
    out, lse = la.decode(qkv.cuda(), w.NH)
    torch.cuda.synchronize()
    ro, rl = _decode_ref(oracle_mod, qkv, w.NH)
    assert_close(out.cpu(), ro, dtype, "decode out")
    assert_close(lse.cpu(), rl, dtype, "decode lse")


def test_decode_reads_only_the_last_query_row(la):
    B, T, C, NH = 2, 333, 256, 4
    qkv, _ = make_inputs(B, T, C, "f32", seed=77)
    a = la.decode(qkv.cuda(), NH)
    b = la.decode(qkv.cuda(), NH)
    q2 = qkv.clone()
    q2[:, :T - 1, :C] = float("nan")          # queries of earlier rows are never read
    c = la.decode(q2.cuda(), NH)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def _parts(oracle_mod, qkv, NH, causal, edges):
    T = qkv.shape[1]
    outs, lses = [], []
    for a, b in zip(edges, edges[1:]):
        o, l = oracle_mod.forward_block(qkv, NH, causal, 0, T, a, b)
        outs.append(o)
        lses.append(l)
    o = torch.from_numpy(np.stack(outs)).float().contiguous()
    l = torch.from_numpy(np.stack(lses)).float().contiguous()
    return o, l


MERGE_CASES = [
    ((1, 40, 64, 4), True, (0, 13, 40)),
    ((2, 100, 256, 4), True, (0, 1, 50, 64, 100)),
    ((2, 100, 256, 4), False, (0, 33, 100)),
    ((1, 70, 512, 4), True, (0, 64, 70)),
    ((3, 17, 128, 4), False, (0, 17)),          # one part: the identity
]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape,causal,edges", MERGE_CASES)
def test_merge_recovers_forward(la, oracle_mod, shape, causal, edges, out_dtype):
    B, T, C, NH = shape
    _case(f"merge {out_dtype} B{B} T{T} C{C} NH{NH} causal={causal} edges={edges}")
    qkv, _ = make_inputs(B, T, C, "f32", seed=600 + T)
    o_parts, l_parts = _parts(oracle_mod, qkv, NH, causal, edges)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(out_dtype, torch.float32)
    out, lse = la.merge(o_parts.cuda(), l_parts.cuda(), tdt)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.forward(qkv, NH, causal)
    assert_close(out.cpu(), ro, out_dtype, "merged out")
    assert_close(lse.cpu(), rl, "f32", "merged lse")


def test_merge_rows_without_keys(la, oracle_mod):
    """Causal rows before the only part's first key: out 0 and lse -inf."""
    B, T, C, NH = 1, 30, 64, 4
    qkv, _ = make_inputs(B, T, C, "f32", seed=71)
    o_parts, l_parts = _parts(oracle_mod, qkv, NH, True, (10, 30))
    out, lse = la.merge(o_parts.cuda(), l_parts.cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.all(out[:, :10] == 0) and torch.all(torch.isneginf(lse[:, :, :10]))
    ro, rl = oracle_mod.forward_block(qkv, NH, True, 0, T, 10, 30)
    assert_close(out[:, 10:], ro[:, 10:], "f32", "out")
    assert_close(lse[:, :, 10:], rl[:, :, 10:], "f32", "lse")


def test_decode_many_ranges(la, oracle_mod):
    """257 ranges of 128 keys merged for a single head (one workgroup per
    range, more ranges than a workgroup has threads)."""
    B, T, C, NH = 1, 128 * 257, 16, 1
    _case(f"decode f32 B{B} T{T} C{C} NH{NH} (257 ranges)")
    qkv, _ = make_inputs(B, T, C, "f32", seed=81)
    out, lse = la.decode(qkv.cuda(), NH)
    torch.cuda.synchronize()
    ro, rl = _decode_ref(oracle_mod, qkv, NH)
    assert_close(out.cpu(), ro, "f32", "decode out")
    assert_close(lse.cpu(), rl, "f32", "decode lse")


def test_decode_calls_in_a_row(la, oracle_mod):
    """The partial results share the library workspace with the backward's
    D: alternating shapes, with a backward in between, give the same bits
    and the oracle's values each time."""
    _case("decode calls in a row")
    qa, _ = make_inputs(4, 500, 256, "f32", seed=82)
    qb, db = make_inputs(2, 300, 512, "f32", seed=83)
    qa_, qb_ = qa.cuda(), qb.cuda()
    a1 = la.decode(qa_, 4)
    b1 = la.decode(qb_, 8)
    o, l = la.forward(qb_, 8, True)
    la.backward(db.cuda(), qb_, o, l, 8, True)
    a2 = la.decode(qa_, 4)
    b2 = la.decode(qb_, 8)
    torch.cuda.synchronize()
    for x, y in zip(a1 + b1, a2 + b2):
        assert torch.equal(x, y)
    ro, rl = _decode_ref(oracle_mod, qa, 4)
    assert_close(a2[0].cpu(), ro, "f32", "decode out")
    ro, rl = _decode_ref(oracle_mod, qb, 8)
    assert_close(b2[0].cpu(), ro, "f32", "decode out")


def test_decode_graph_replays(la):
    """A captured decode (range kernel and merge kernel) replayed three
    times, with eager decodes of another shape in between, gives the eager
    bits each time."""
    _case("decode under graph capture")
    qa, _ = make_inputs(4, 700, 256, "bf16", seed=85)
    qb, _ = make_inputs(2, 300, 512, "bf16", seed=86)
    qa_, qb_ = qa.cuda(), qb.cuda()
    out = torch.empty((4, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((4, 4), device="cuda")
    la.attn_decode_bf16(out, lse, qa_, 4, 700, 256, 4)   # eager: sizes the workspace
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.attn_decode_bf16(out, lse, qa_, 4, 700, 256, 4)
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {r}"
        la.decode(qb_, 8)
        torch.cuda.synchronize()
