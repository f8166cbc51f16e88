"""bench.py's accounting on the CPU: the per-kernel flop counts add up to
the useful 14 * hs * pairs * B * NH for the fp32 attn_backward (one kernel
for dK, dV and dQ: 4 + 10) and for the fp32 dS block store order (whose dQ
kernel reads the stored dS: 4 + 8 + 2), and to 18 * hs * pairs * B * NH
for the recompute order that the 16-bit attn_backward_* and the fp32
stages attn_backward_dq + attn_backward_dkdv run (whose dQ kernel
recomputes S and dP: 4 + 8 + 6), and the compulsory HBM bytes
match the figures worked out by hand for the five workloads (forward: qkv
read, out and lse written; backward: qkv, out, dout, lse read, D written and
read, dqkv written)."""
import pytest

import bench
from workloads import WORKLOADS


@pytest.mark.parametrize("key", sorted(WORKLOADS))
@pytest.mark.parametrize("dtype", ["f32", "f32_ds", "f32_rc", "bf16"])
def test_kernel_flops_add_up_to_the_step(key, dtype):
    w = WORKLOADS[key]
    kf = bench.kernel_flops(w, dtype)
    unit = w.hs * w.pairs * w.B * w.NH
    assert w.flops_fwd + w.flops_bwd == 14 * unit
    staged = {k: v for k, v in kf.items() if k != "bwd_short"}
    assert sum(staged.values()) == (14 if dtype in ("f32", "f32_ds") else 18) * unit
    assert kf["fwd"] == w.flops_fwd
    if dtype == "bf16":   # the one-kernel short-sequence backward: five contractions
        assert kf["bwd_short"] == w.flops_bwd == 10 * unit


def test_short_backward_rule():
    """The step times the fused 16-bit backward as one stage exactly for the
    shapes where the library runs its one-workgroup-per-head kernel."""
    assert bench.short_backward(WORKLOADS[4], "bf16")          # ViT-B/16, T = 196, hs = 64
    assert not bench.short_backward(WORKLOADS[3], "bf16")      # GPT-2 layer, T = 1024
    assert not bench.short_backward(WORKLOADS[5], "bf16")      # long context, hs = 128
    assert not bench.short_backward(WORKLOADS[4], "f32")       # 16-bit kernels only
    assert bench.short_backward(WORKLOADS[2], "bf16")          # T = 256, hs = 64
    assert bench.short_backward(WORKLOADS[1], "bf16")          # T = 64, hs = 16


def test_compulsory_bytes_by_hand():
    # GPT-2 layer B8 T1024 C768 NH12: B*T*C = 6291456 elements, B*NH*T = 98304 rows
    io, rows = 6291456, 98304
    assert bench.compulsory_bytes(WORKLOADS[3], "f32") == (16 * io + 4 * rows,
                                                          32 * io + 12 * rows)
    assert bench.compulsory_bytes(WORKLOADS[3], "f32") == (101056512, 202506240)
    assert bench.compulsory_bytes(WORKLOADS[3], "bf16") == (50724864, 101842944)
    # ViT-B/16 B128 T196 C768 NH12, bf16
    assert bench.compulsory_bytes(WORKLOADS[4], "bf16") == (155344896, 311894016)
    # long context B1 T8192 C2048 NH16, bf16
    assert bench.compulsory_bytes(WORKLOADS[5], "bf16") == (134742016, 270008320)


def test_hbm_report_rates():
    r = bench.hbm_report(WORKLOADS[3], "f32", 0.1, 0.2)
    assert r["gbs_fwd"] == pytest.approx(101056512 / 1e-4 / 1e9, rel=1e-3)
    assert r["frac_hbm_peak_step"] == pytest.approx((101056512 + 202506240) / 3e-4 / 8e12,
                                                    abs=1e-4)


def test_gpus_above_one_is_refused():
    import subprocess
    import sys
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                         text=True, cwd=bench.ROOT, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr
