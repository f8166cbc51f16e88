"""Seeded synthetic inputs for the attention path.

This module only draws random numbers and names shapes: it holds none of the
method's arithmetic, so both the HIP library's tests/benchmark and the CPU
oracle can take their inputs from here without sharing any computation.

Recipe (the same bytes go to the GPU and to the oracle):
  * qkv of shape (B, T, 3C) and dout of shape (B, T, C) are drawn on the host
    with ``torch.Generator('cpu').manual_seed(seed)`` and ``torch.randn`` in
    float32, dout then multiplied by its standard deviation (1 or 0.1);
  * the bf16 workloads round those float32 samples to bfloat16 (and the fp16
    runs to IEEE half, the fp8 runs to OCP FP8 E4M3) with torch's
    round-to-nearest-even cast; the oracle then sees the rounded values;
  * seeds are 1000 + k for qkv and 2000 + k for dout, for workload k.

The shapes are the ones the pages use: the GPT-2 small attention layer of the
llm.c attention test (C=768, NH=12, T=1024; B=8 here), the ViT-B/16 token
count of the self-attention page (224x224 image, 16x16 patches -> 196 tokens,
width 768, 12 heads), plus a tiny, a small and a long-context case.  Synthetic
N(0,1) activations stand in for real ones; no dataset or weights are needed.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    key: int          # 1..5
    name: str
    B: int
    T: int
    C: int
    NH: int
    dtype: str        # "f32" or "bf16"
    causal: bool
    dout_std: float
    materialized: bool = False

    @property
    def hs(self) -> int:
        return self.C // self.NH

    @property
    def pairs(self) -> int:
        """Unmasked (query, key) pairs per head."""
        return self.T * (self.T + 1) // 2 if self.causal else self.T * self.T

    @property
    def flops_fwd(self) -> int:
        return 4 * self.hs * self.pairs * self.B * self.NH

    @property
    def flops_bwd(self) -> int:
        return 10 * self.hs * self.pairs * self.B * self.NH

    def label(self) -> str:
        return (f"B{self.B} T{self.T} C{self.C} NH{self.NH} "
                f"{'causal' if self.causal else 'non-causal'} {self.dtype}")


WORKLOADS = {
    1: Workload(1, "tiny", 1, 64, 64, 4, "f32", True, 1.0),
    2: Workload(2, "small", 4, 256, 256, 4, "f32", True, 1.0, materialized=True),
    3: Workload(3, "gpt2-small-layer", 8, 1024, 768, 12, "f32", True, 1.0),
    4: Workload(4, "vit-b16", 128, 196, 768, 12, "bf16", False, 0.1),
    5: Workload(5, "long-context", 1, 8192, 2048, 16, "bf16", True, 0.1),
}


def randn(shape, seed: int, std: float = 1.0, dtype: str = "f32") -> torch.Tensor:
    """float32 N(0, std^2) samples from a seeded CPU generator, optionally
    rounded to bfloat16, float16 or float8 E4M3 (round to nearest even)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f16":
        return x.to(torch.float16)
    if dtype == "fp8":
        return x.to(torch.float8_e4m3fn)
    if dtype != "f32":
        raise ValueError(dtype)
    return x


def randn_device(shape, seed: int, std: float = 1.0, dtype: str = "f32",
                 device: str = "cuda") -> torch.Tensor:
    """Like randn, drawn on the device with a seeded device generator, for
    inputs too large to draw on the host (the tests copy the slices they
    check back to the host, so the oracle sees the same values)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x = x * std
    return x.to({"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
                 "fp8": torch.float8_e4m3fn}[dtype])


def make_inputs(B: int, T: int, C: int, dtype: str = "f32", seed: int = 0,
                dout_std: float = 1.0):
    """(qkv (B,T,3C), dout (B,T,C)) on the host, seeds `seed` and `seed+1`."""
    qkv = randn((B, T, 3 * C), seed, 1.0, dtype)
    dout = randn((B, T, C), seed + 1, dout_std, dtype)
    return qkv, dout


def workload_inputs(w: Workload, dtype: str | None = None):
    """The seeded inputs of workload `w` (seeds 1000+k and 2000+k)."""
    dt = dtype or w.dtype
    qkv = randn((w.B, w.T, 3 * w.C), 1000 + w.key, 1.0, dt)
    dout = randn((w.B, w.T, w.C), 2000 + w.key, w.dout_std, dt)
    return qkv, dout
