"""attn_backward_noalloc (the fp32 backward with its D scratch in a fixed
device array, for callers that cannot allocate) gives what attn_backward
gives (dk and dv bit for bit, dq up to the order of its atomic sums),
through the C ABI, on two calls in a row, the second with a smaller input;
and again after the first pair, so a stale array from an earlier, larger
call changes nothing."""
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


def _both(la, B, T, C, NH, causal, seed):
    print(f"\n[case] attn_backward_noalloc vs attn_backward B{B} T{T} C{C} NH{NH} "
          f"causal={causal}", flush=True)
    sys.stdout.flush()
    qkv_c, dout_c = make_inputs(B, T, C, "f32", seed=seed)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    c = int(causal)
    out, lse = la.forward(qkv, NH, causal)
    ref = torch.full_like(qkv, float("nan"))
    got = torch.full_like(qkv, float("nan"))
    la.attn_backward(ref, dout, qkv, out, lse, B, T, C, NH, c)
    la.attn_backward_noalloc(got, dout, qkv, out, lse, B, T, C, NH, c)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert_atomic_dq_equal(got, ref, C, "attn_backward_noalloc")


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_equals_attn_backward_twice_second_smaller(la, causal):
    _both(la, 4, 700, 768, 12, causal, seed=91)     # 33600 rows of D
    _both(la, 2, 130, 256, 4, causal, seed=92)      # smaller, ragged
    _both(la, 1, 1, 64, 4, causal, seed=93)         # T = 1


def test_noalloc_at_the_gpt2_layer_and_at_its_limit(la):
    _both(la, 8, 1024, 768, 12, True, seed=94)      # the benchmark's shape
    # B*NH*T = 64*64*1024 = 4194304: the largest D the fixed scratch holds
    _both(la, 64, 1024, 1024, 64, True, seed=95)
    _both(la, 2, 65, 128, 2, True, seed=96)
