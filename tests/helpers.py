"""Shared test helpers: the tolerance check and GPU call wrappers."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances on |gpu - oracle| <= atol + rtol * |oracle|, elementwise.
# fp16 (not in the stated targets) gets ten of its rounding steps, 2^-11 each:
# the same margin over one rounding that the bf16 bound leaves over bf16's 2^-8.
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 2e-2), "f16": (5e-3, 5e-3)}


def assert_close(gpu, ref, dtype: str, what: str):
    """Elementwise check against the oracle; the message reports the max
    absolute and relative errors and the number of violations."""
    atol, rtol = TOL[dtype]
    g = gpu.detach().to("cpu").double().numpy() if hasattr(gpu, "detach") else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in GPU result"
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    nbad = int(bad.sum())
    if nbad:
        idx = np.unravel_index(int(np.argmax(err - (atol + rtol * np.abs(r)))), r.shape)
        rel = err / np.maximum(np.abs(r), 1e-30)
        raise AssertionError(
            f"{what}: {nbad}/{r.size} elements outside atol={atol} rtol={rtol}; "
            f"max abs err {err.max():.3e}, max rel err {rel.max():.3e}; "
            f"worst at {idx}: gpu={g[idx]!r} ref={r[idx]!r}")
    return float(err.max())


def gpu_fwd_bwd(la, qkv_cpu: torch.Tensor, dout_cpu: torch.Tensor, NH: int, causal: bool):
    """Run the fused forward and backward on cuda:0; return CPU tensors
    (out, lse, dqkv)."""
    qkv = qkv_cpu.to("cuda")
    dout = dout_cpu.to("cuda")
    out, lse = la.forward(qkv, NH, causal)
    dqkv = la.backward(dout, qkv, out, lse, NH, causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), dqkv.cpu()


def head_view(x, b: int, h: int, NH: int, packed: bool):
    """Slice head (b, h) of a packed (B,T,3C) or (B,T,C) array the same way
    oracle.head_slice does (pure indexing), for comparisons."""
    x = x.detach().cpu().double().numpy() if hasattr(x, "detach") else np.asarray(x)
    if packed:
        C = x.shape[2] // 3
        hs = C // NH
        return np.concatenate([x[b:b + 1, :, p * C + h * hs:p * C + (h + 1) * hs]
                               for p in range(3)], axis=2)
    C = x.shape[2]
    hs = C // NH
    return x[b:b + 1, :, h * hs:(h + 1) * hs]
