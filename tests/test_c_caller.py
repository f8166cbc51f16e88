"""libattn from plain C (tests/c_caller/attn_c_caller.c): the program
includes include/libattn.h, allocates with hipMalloc, runs the fp32 forward
and backward and compares every element with the fp64 oracle.  On the CPU it
must compile and link against libattn.so, liboracle.so and the HIP runtime;
on the GPU it must run and report every case within the fp32 bounds."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_caller", "attn_c_caller.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out_dir) -> str:
    from transformer_causal_head_attn_amd import LIB_PATH
    import oracle
    lib_oracle = oracle.build()
    if not os.path.exists(LIB_PATH):
        pytest.fail(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    exe = os.path.join(str(out_dir), "attn_c_caller")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-o", exe, SRC, LIB_PATH, lib_oracle, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-lm", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-Wl,-rpath," + os.path.dirname(LIB_PATH), "-Wl,-rpath," + os.path.dirname(lib_oracle)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_c_caller_compiles_and_links(tmp_path):
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_caller_runs_against_the_oracle(tmp_path):
    exe = _build(tmp_path)
    print("\n[case] C caller: fp32 forward + backward from C against the oracle", flush=True)
    sys.stdout.flush()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(res.stdout[-3000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-2000:]
    assert "c caller ok" in res.stdout
