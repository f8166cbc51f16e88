"""Batches whose packed tensors pass 2^31 elements (and 2^32 bytes): every
offset into qkv, out, lse and dqkv for the last sequences needs 64-bit
arithmetic.  The inputs are drawn on the device (seeded); the heads checked
are copied back and compared with the oracle element by element."""
import numpy as np
import pytest
import torch

from helpers import assert_close
from workloads import randn_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import transformer_causal_head_attn_amd as m
    m.load()
    return m


def _head(x, b, h, NH, packed):
    """Head (b, h) of a device tensor as a host (1, T, 3hs) or (1, T, hs) array."""
    C = x.shape[2] // 3 if packed else x.shape[2]
    hs = C // NH
    if packed:
        parts = [x[b:b + 1, :, p * C + h * hs:p * C + (h + 1) * hs] for p in range(3)]
        return torch.cat(parts, dim=2).cpu()
    return x[b:b + 1, :, h * hs:(h + 1) * hs].cpu()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_offsets_past_32_bits(la, oracle_mod, dtype):
    B, T, C, NH = 1100, 1024, 768, 12        # B*T*3C = 2.6e9 elements
    print(f"\n[case] {dtype} B{B} T{T} C{C} NH{NH}", flush=True)
    assert B * T * 3 * C > 2 ** 31
    qkv = randn_device((B, T, 3 * C), 91, 1.0, dtype)
    dout = randn_device((B, T, C), 92, 1.0, dtype)
    out, lse = la.forward(qkv, NH, True)
    dqkv = la.backward(dout, qkv, out, lse, NH, True)
    dec_out, dec_lse = la.decode(qkv, NH)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (777, 5), (B - 1, NH - 1)]:
        qs = _head(qkv, b, h, NH, True)
        ds = _head(dout, b, h, NH, False)
        ro, rl = oracle_mod.forward(qs, 1, True)
        rd = oracle_mod.backward(qs, ds, 1, True)
        assert_close(_head(out, b, h, NH, False), ro, dtype, f"out head {(b, h)}")
        assert_close(lse[b:b + 1, h:h + 1].cpu(), rl, dtype, f"lse head {(b, h)}")
        assert_close(_head(dqkv, b, h, NH, True), rd, dtype, f"dqkv head {(b, h)}")
        hs = C // NH
        assert_close(dec_out[b, h * hs:(h + 1) * hs].cpu(), ro[0, T - 1], dtype, f"decode head {(b, h)}")
        assert_close(dec_lse[b, h].cpu(), rl[0, 0, T - 1], dtype, f"decode lse head {(b, h)}")
    del qkv, dout, out, lse, dqkv
    torch.cuda.empty_cache()


def test_fp8_forward_offsets_past_32_bits(la, oracle_mod):
    """fp8 qkv of more than 2^32 bytes (one byte per element): the last
    sequences' offsets need 64-bit arithmetic in the fp8 forward too."""
    from helpers import LSE_ATOL_FP8, assert_close_scaled
    B, T, C, NH = 1850, 1024, 768, 12        # B*T*3C = 4.4e9 bytes
    print(f"\n[case] fp8 forward B{B} T{T} C{C} NH{NH}", flush=True)
    assert B * T * 3 * C > 2 ** 32
    qkv = randn_device((B, T, 3 * C), 93, 1.0, "fp8")
    out, lse = la.forward_fp8(qkv, NH, True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1299, 7), (B - 1, NH - 1)]:
        qs = _head(qkv, b, h, NH, True)
        ro, rl = oracle_mod.forward(qs, 1, True)
        assert_close_scaled(_head(out, b, h, NH, False), ro, "fp8", f"out head {(b, h)}", 1, "rows")
        err = np.abs(lse[b:b + 1, h:h + 1].cpu().double().numpy() - rl).max()
        assert err <= LSE_ATOL_FP8, f"lse head {(b, h)}: {err}"
    del qkv, out, lse
    torch.cuda.empty_cache()
