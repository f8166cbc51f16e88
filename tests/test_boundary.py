"""The C ABI of libattn on a host without a GPU: the library loads, exports
every entry point its header declares, and rejects bad arguments with the
documented status before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import transformer_causal_head_attn_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:attn|layernorm)_\w+)\s*\(", src)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(la.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = la.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared_functions():
        assert name in syms, name


def test_header_compiles_as_c():
    src = '#include "libattn.h"\nint main(void){return attn_set_stream(0);}\n'
    res = subprocess.run(["gcc", "-fsyntax-only", "-std=c99", "-Wall", "-Werror",
                          "-I", os.path.dirname(HEADER), "-x", "c", "-"],
                         input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


# Fake, aligned, non-overlapping addresses: argument checks never dereference
# them, and every case below is rejected before any HIP call.
BASE = 1 << 40
STEP = 1 << 36


def ptrs(n):
    return [ctypes.c_void_p(BASE + i * STEP) for i in range(n)]


def call(name, nptr, B, T, C, NH, causal, override=None):
    lib = la.load()
    p = ptrs(nptr)
    if override:
        for i, v in override.items():
            p[i] = ctypes.c_void_p(v)
    rc = getattr(lib, name)(*p, B, T, C, NH, causal)
    return rc, lib.attn_last_error().decode()


ENTRY = [("attn_forward", 3), ("attn_backward", 5), ("attn_backward_noalloc", 5),
         ("attn_forward_bf16", 3),
         ("attn_backward_bf16", 5), ("attn_forward_materialized", 4),
         ("attn_backward_materialized", 6),
         ("attn_backward_dkdv", 5), ("attn_backward_dq", 6),
         ("attn_backward_dkdv_bf16", 5), ("attn_backward_dq_bf16", 6),
         ("attn_forward_f16", 3), ("attn_backward_f16", 5),
         ("attn_backward_dkdv_f16", 5), ("attn_backward_dq_f16", 6),
         ("attn_backward_dkdv_ds", 6), ("attn_backward_dq_ds", 3),
         ("attn_backward_dkdvdq", 5), ("attn_forward_fp8", 3)]
STAGE0 = [("attn_backward_preprocess", 3), ("attn_backward_preprocess_bf16", 3),
          ("attn_backward_preprocess_f16", 3), ("attn_backward_prepare", 4)]


@pytest.mark.parametrize("name,nptr", ENTRY)
@pytest.mark.parametrize("dims,code", [
    ((0, 64, 64, 4, 1), la.ATTN_EINVAL),       # B < 1
    ((1, 0, 64, 4, 1), la.ATTN_EINVAL),        # T < 1
    ((1, 64, 64, 0, 1), la.ATTN_EINVAL),       # NH < 1
    ((1, 64, 3, 4, 1), la.ATTN_EINVAL),        # C < NH
    ((1, 64, 66, 4, 1), la.ATTN_EINVAL),       # C % NH != 0
    ((1, 64, 64, 4, 2), la.ATTN_EINVAL),       # causal not 0/1
    ((1, 64, 64, 4, -1), la.ATTN_EINVAL),
    ((1, 64, 96, 4, 1), la.ATTN_EUNSUPPORTED),  # hs = 24
    ((1, 64, 256, 1, 1), la.ATTN_EUNSUPPORTED),  # hs = 256
    ((1, 64, 8, 1, 0), la.ATTN_EUNSUPPORTED),    # hs = 8
])
def test_bad_dimensions(name, nptr, dims, code):
    rc, msg = call(name, nptr, *dims)
    assert rc == code, msg
    assert msg


@pytest.mark.parametrize("name,nptr", ENTRY)
def test_null_pointers(name, nptr):
    for i in range(nptr):
        rc, msg = call(name, nptr, 1, 64, 64, 4, 1, override={i: 0})
        assert rc == la.ATTN_EINVAL and "NULL" in msg


@pytest.mark.parametrize("name,nptr", ENTRY)
def test_misaligned_pointer(name, nptr):
    rc, msg = call(name, nptr, 1, 64, 64, 4, 1, override={0: BASE + 4})
    assert rc == la.ATTN_EINVAL and "aligned" in msg


@pytest.mark.parametrize("name,nptr", ENTRY)
def test_output_overlapping_input(name, nptr):
    # put the last argument (an input) 16 bytes into the first (an output)
    rc, msg = call(name, nptr, 1, 64, 64, 4, 1, override={nptr - 1: BASE + 16})
    assert rc == la.ATTN_EINVAL and "overlaps" in msg


@pytest.mark.parametrize("name,nptr", STAGE0)
def test_preprocess_arguments(name, nptr):
    lib = la.load()
    p = ptrs(nptr)
    assert getattr(lib, name)(*p, 1, 64, 64, 0) == la.ATTN_EINVAL
    assert getattr(lib, name)(*p, 1, 64, 66, 4) == la.ATTN_EINVAL
    assert getattr(lib, name)(*p, 1, 64, 96, 4) == la.ATTN_EUNSUPPORTED
    p[0] = ctypes.c_void_p(0)
    assert getattr(lib, name)(*p, 1, 64, 64, 4) == la.ATTN_EINVAL
    p = ptrs(nptr)
    p[2] = ctypes.c_void_p(BASE + 16)   # out overlaps the D output
    assert getattr(lib, name)(*p, 1, 64, 64, 4) == la.ATTN_EINVAL


def test_too_large_for_32bit_offsets():
    rc, msg = call("attn_forward", 3, 1, 1 << 20, 1024, 16, 1)
    assert rc == la.ATTN_EINVAL and "32-bit" in msg
    rc, msg = call("attn_forward_materialized", 4, 1, 1 << 16, 64, 4, 1)
    assert rc == la.ATTN_EINVAL and "T*T" in msg
    # T*3C fits in 31 bits, but one 64-row tile of fp32 rows does not fit 32-bit byte offsets
    C = 64 * 98304
    for name, nptr in [("attn_forward", 3), ("attn_backward_bf16", 5)]:
        rc, msg = call(name, nptr, 1, 1, C, C // 64, 1)
        assert rc == la.ATTN_EINVAL and "buffer offset" in msg


def test_ds_store_bytes():
    """One 64x64 fp32 block per kept (query tile, key tile) pair and head."""
    blk = 64 * 64 * 4
    assert la.attn_backward_ds_bytes(8, 1024, 768, 12, 1) == 96 * (16 * 17 // 2) * blk
    assert la.attn_backward_ds_bytes(8, 1024, 768, 12, 0) == 96 * 16 * 16 * blk
    assert la.attn_backward_ds_bytes(1, 65, 64, 4, 1) == 4 * 3 * blk
    assert la.attn_backward_ds_bytes(2, 1, 128, 2, 0) == 4 * blk
    assert la.attn_backward_ds_bytes(1, 64, 66, 4, 1) == 0
    assert la.attn_backward_ds_bytes(1, 64, 96, 4, 1) == 0   # hs = 24
    assert la.attn_backward_ds_bytes(0, 64, 64, 4, 1) == 0


def test_ds_store_overlaps():
    """The dS store's whole extent is checked against the other tensors."""
    size = la.attn_backward_ds_bytes(1, 64, 64, 4, 1)
    # dS (argument 1) runs into D (argument 5)
    rc, msg = call("attn_backward_dkdv_ds", 6, 1, 64, 64, 4, 1,
                   override={5: BASE + STEP + size - 16})
    assert rc == la.ATTN_EINVAL and "overlaps" in msg
    # dS (argument 1) starts inside dqkv (argument 0)
    for name, nptr in (("attn_backward_dkdv_ds", 6), ("attn_backward_dq_ds", 3)):
        rc, msg = call(name, nptr, 1, 64, 64, 4, 1, override={1: BASE + 16})
        assert rc == la.ATTN_EINVAL and "overlaps" in msg, (name, msg)
    # dqkv (argument 0) ends inside dS
    rc, msg = call("attn_backward_dq_ds", 3, 1, 64, 64, 4, 1,
                   override={0: BASE + STEP - 64 * 192 * 4 + 16})
    assert rc == la.ATTN_EINVAL and "overlaps" in msg


def test_forced_workspace_failure():
    """ATTN_TEST_FAIL_ALLOC=1 makes the backward's workspace allocation fail
    with ATTN_EHIP before any HIP call (run in a child process so the
    environment variable is read fresh)."""
    code = (
        "import ctypes, transformer_causal_head_attn_amd as la\n"
        "lib = la.load()\n"
        "p = [ctypes.c_void_p((1 << 40) + i * (1 << 36)) for i in range(5)]\n"
        "rc = lib.attn_backward(*p, 1, 64, 64, 4, 1)\n"
        "print(rc, lib.attn_last_error().decode())\n"
    )
    env = dict(os.environ, ATTN_TEST_FAIL_ALLOC="1", PYTHONPATH=ROOT)
    res = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=120)
    assert res.returncode == 0, res.stderr
    rc, msg = res.stdout.split(" ", 1)
    assert int(rc) == la.ATTN_EHIP and "forced" in msg


def test_last_error_cleared_by_success():
    lib = la.load()
    call("attn_forward", 3, 0, 1, 1, 1, 1)
    assert la.attn_last_error()
    assert lib.attn_set_stream(None) == la.ATTN_OK
    assert la.attn_last_error() == ""


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 64, 192)
    with pytest.raises(ValueError):
        la.forward(x, 4, True)


DECODE = ["attn_decode", "attn_decode_bf16", "attn_decode_f16"]
MERGE = ["attn_merge", "attn_merge_bf16", "attn_merge_f16"]


@pytest.mark.parametrize("name", DECODE)
def test_decode_arguments(name):
    lib = la.load()
    fn = getattr(lib, name)
    p = ptrs(3)
    assert fn(*p, 0, 64, 64, 4) == la.ATTN_EINVAL          # B < 1
    assert fn(*p, 1, 0, 64, 4) == la.ATTN_EINVAL           # T < 1
    assert fn(*p, 1, 64, 66, 4) == la.ATTN_EINVAL          # C % NH
    assert fn(*p, 1, 64, 96, 4) == la.ATTN_EUNSUPPORTED    # hs = 24
    for i in range(3):
        q = ptrs(3)
        q[i] = ctypes.c_void_p(0)
        assert fn(*q, 1, 64, 64, 4) == la.ATTN_EINVAL
        assert "NULL" in lib.attn_last_error().decode()
    q = ptrs(3)
    q[1] = ctypes.c_void_p(BASE + 4)                       # lse overlaps out (B*C*esize bytes)
    assert fn(*q, 1, 64, 64, 4) == la.ATTN_EINVAL
    q = ptrs(3)
    q[2] = ctypes.c_void_p(BASE + STEP + 2)                # misaligned qkv
    assert fn(*q, 1, 64, 64, 4) == la.ATTN_EINVAL


@pytest.mark.parametrize("name", MERGE)
def test_merge_arguments(name):
    lib = la.load()
    fn = getattr(lib, name)
    p = ptrs(4)
    assert fn(*p, 0, 1, 8, 64, 4) == la.ATTN_EINVAL        # nparts < 1
    assert "nparts" in lib.attn_last_error().decode()
    assert fn(*p, 2, 0, 8, 64, 4) == la.ATTN_EINVAL        # B < 1
    assert fn(*p, 2, 1, 8, 64, 3) == la.ATTN_EINVAL        # C % NH
    assert fn(*p, 2, 1, 8, 48, 1) == la.ATTN_EUNSUPPORTED  # hs = 48
    for i in range(4):
        q = ptrs(4)
        q[i] = ctypes.c_void_p(0)
        assert fn(*q, 2, 1, 8, 64, 4) == la.ATTN_EINVAL
    q = ptrs(4)
    q[2] = ctypes.c_void_p(BASE + 16)                      # o_parts inside out
    assert fn(*q, 2, 1, 8, 64, 4) == la.ATTN_EINVAL
    assert "overlaps" in lib.attn_last_error().decode()


def test_forced_workspace_failure_decode():
    """attn_decode keeps its partial results in the workspace: the forced
    allocation failure reaches it too, before any HIP call."""
    code = (
        "import ctypes, transformer_causal_head_attn_amd as la\n"
        "lib = la.load()\n"
        "p = [ctypes.c_void_p((1 << 40) + i * (1 << 36)) for i in range(3)]\n"
        "rc = lib.attn_decode(*p, 1, 64, 64, 4)\n"
        "print(rc, lib.attn_last_error().decode())\n"
    )
    env = dict(os.environ, ATTN_TEST_FAIL_ALLOC="1", PYTHONPATH=ROOT)
    res = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=120)
    assert res.returncode == 0, res.stderr
    rc, msg = res.stdout.split(" ", 1)
    assert int(rc) == la.ATTN_EHIP and "forced" in msg


def test_error_state_is_per_thread():
    """attn_last_error and the stream are thread-local: a failure in one
    thread leaves another thread's message untouched."""
    import threading
    lib = la.load()
    seen = {}
    ready = threading.Event()
    go = threading.Event()

    def failing():
        call("attn_forward", 3, 0, 64, 64, 4, 1)       # B < 1
        seen["a"] = lib.attn_last_error().decode()
        ready.set()

    def clean():
        assert lib.attn_set_stream(None) == la.ATTN_OK  # clears this thread's message
        go.wait(timeout=30)
        seen["b"] = lib.attn_last_error().decode()

    tb = threading.Thread(target=clean)
    tb.start()
    ta = threading.Thread(target=failing)
    ta.start()
    ready.wait(timeout=30)
    go.set()
    ta.join(timeout=30)
    tb.join(timeout=30)
    assert "B, T and NH" in seen["a"]
    assert seen["b"] == ""


LN = [("layernorm_forward", 6), ("layernorm_forward_bf16", 6), ("layernorm_forward_f16", 6),
      ("layernorm_backward", 8), ("layernorm_backward_bf16", 8), ("layernorm_backward_f16", 8)]


@pytest.mark.parametrize("name,nptr", LN)
def test_layernorm_arguments(name, nptr):
    lib = la.load()
    fn = getattr(lib, name)
    p = ptrs(nptr)
    assert fn(*p, 0, 768) == la.ATTN_EINVAL                # N < 1
    assert fn(*p, 8, 0) == la.ATTN_EINVAL                  # C < 1
    assert "N and C" in lib.attn_last_error().decode()
    for i in range(nptr):
        q = ptrs(nptr)
        q[i] = ctypes.c_void_p(0)
        assert fn(*q, 8, 768) == la.ATTN_EINVAL
        assert "NULL" in lib.attn_last_error().decode()
        q = ptrs(nptr)
        q[i] = ctypes.c_void_p(BASE + i * STEP + 4)
        assert fn(*q, 8, 768) == la.ATTN_EINVAL
        assert "aligned" in lib.attn_last_error().decode()
    for o in range(3):                                     # each output inside each input
        for j in range(3, nptr):
            q = ptrs(nptr)
            q[o] = ctypes.c_void_p(BASE + j * STEP + 16)
            assert fn(*q, 8, 768) == la.ATTN_EINVAL
            assert "overlaps" in lib.attn_last_error().decode()
    q = ptrs(nptr)
    q[1] = ctypes.c_void_p(BASE + 16)                      # second output inside the first
    assert fn(*q, 8, 768) == la.ATTN_EINVAL


def test_forced_workspace_failure_layernorm_backward():
    """The LayerNorm backward keeps partial column sums in the workspace:
    the forced allocation failure reaches it before any HIP call."""
    code = (
        "import ctypes, transformer_causal_head_attn_amd as la\n"
        "lib = la.load()\n"
        "p = [ctypes.c_void_p((1 << 40) + i * (1 << 36)) for i in range(8)]\n"
        "rc = lib.layernorm_backward(*p, 8, 768)\n"
        "print(rc, lib.attn_last_error().decode())\n"
    )
    env = dict(os.environ, ATTN_TEST_FAIL_ALLOC="1", PYTHONPATH=ROOT)
    res = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=120)
    assert res.returncode == 0, res.stderr
    rc, msg = res.stdout.split(" ", 1)
    assert int(rc) == la.ATTN_EHIP and "forced" in msg


def test_noalloc_rejects_shapes_past_its_fixed_scratch():
    """attn_backward_noalloc holds D (B*NH*T floats) in a fixed array of
    4194304 floats: a larger shape is refused before any HIP call."""
    rc, msg = call("attn_backward_noalloc", 5, 1100, 1024, 768, 12, 1)
    assert rc == la.ATTN_EINVAL and "fixed scratch" in msg
    rc, msg = call("attn_backward_noalloc", 5, 342, 1024, 768, 12, 1)   # 4202496 rows
    assert rc == la.ATTN_EINVAL and "fixed scratch" in msg


def _splitkv(name, B, T, C, NH, causal, kv_chunk, override=None):
    lib = la.load()
    p = ptrs(4)
    if override:
        for i, v in override.items():
            p[i] = ctypes.c_void_p(v)
    rc = getattr(lib, name)(*p, B, T, C, NH, causal, kv_chunk)
    return rc, lib.attn_last_error().decode()


@pytest.mark.parametrize("name", ["attn_forward_splitkv_bf16", "attn_forward_splitkv_f16"])
def test_splitkv_argument_errors(name):
    for chunk in (-64, 100, 32):
        rc, msg = _splitkv(name, 1, 8192, 256, 2, 1, chunk)
        assert rc == la.ATTN_EINVAL and "kv_chunk" in msg
    for i in range(4):
        rc, msg = _splitkv(name, 1, 8192, 256, 2, 1, 2048, override={i: 0})
        assert rc == la.ATTN_EINVAL and "NULL" in msg
    rc, msg = _splitkv(name, 1, 8192, 96, 4, 1, 2048)
    assert rc == la.ATTN_EUNSUPPORTED


def test_splitkv_work_bytes():
    lib = la.load()
    # two heads of the long-context shape, 2048-key chunks: 4 parts of
    # (B*T*C + B*NH*T) floats
    B, T, C, NH = 1, 8192, 256, 2
    assert lib.attn_forward_splitkv_bytes(B, T, C, NH, 1, 2048) == 4 * 4 * (B * T * C + B * NH * T)
    # a ragged T: ceil(ceil(1000/64)/3) = 6 parts of 192 keys
    assert lib.attn_forward_splitkv_bytes(2, 1000, 128, 2, 0, 192) == 6 * 4 * (2 * 1000 * 128 + 2 * 2 * 1000)
    # a chunk covering every key: no split, no work
    assert lib.attn_forward_splitkv_bytes(B, T, C, NH, 1, 8192) == 0
    assert lib.attn_forward_splitkv_bytes(B, T, C, NH, 1, 1 << 20) == 0
    # rejected arguments: 0
    assert lib.attn_forward_splitkv_bytes(B, T, C, NH, 1, 100) == 0
    assert lib.attn_forward_splitkv_bytes(B, T, 96, 4, 1, 2048) == 0


def test_backward_splitkv_work_bytes_and_errors():
    lib = la.load()
    B, T, C, NH = 1, 8192, 256, 2
    d = B * NH * T   # a multiple of 64 already
    assert lib.attn_backward_splitkv_bytes(B, T, C, NH, 1, 2048) == 4 * (d + 3 * 4 * B * T * C)
    # no split: D only (rounded up to 64 floats)
    assert lib.attn_backward_splitkv_bytes(2, 100, 64, 4, 1, 128) == 4 * 832
    assert lib.attn_backward_splitkv_bytes(B, T, C, NH, 1, 100) == 0
    p = ptrs(6)
    for name in ("attn_backward_splitkv_bf16", "attn_backward_splitkv_f16"):
        rc = getattr(lib, name)(*p, B, T, C, NH, 1, 96)
        assert rc == la.ATTN_EINVAL and b"kv_chunk" in lib.attn_last_error()
        q = list(p)
        q[5] = ctypes.c_void_p(0)
        rc = getattr(lib, name)(*q, B, T, C, NH, 1, 2048)
        assert rc == la.ATTN_EINVAL and b"NULL" in lib.attn_last_error()


@pytest.mark.parametrize("name,nptr", [("attn_qkv_projection", 4), ("attn_qkv_projection_bf16", 4),
                                       ("attn_out_projection", 5), ("attn_out_projection_bf16", 5)])
def test_projection_argument_errors(name, nptr):
    lib = la.load()
    f = getattr(lib, name)
    kmul = 8 if name.endswith("bf16") else 4
    assert f(*ptrs(nptr), 0, 64, 64) == la.ATTN_EINVAL
    assert f(*ptrs(nptr), 64, kmul + 2, 64) == la.ATTN_EINVAL      # K not a multiple
    assert b"multiple" in lib.attn_last_error()
    assert f(*ptrs(nptr), 64, 64, 66) == la.ATTN_EINVAL            # N % 4
    for i in range(nptr):
        p = ptrs(nptr)
        p[i] = ctypes.c_void_p(0)
        assert f(*p, 64, 64, 64) == la.ATTN_EINVAL and b"NULL" in lib.attn_last_error()
    p = ptrs(nptr)
    p[0] = ctypes.c_void_p(BASE + 8)
    assert f(*p, 64, 64, 64) == la.ATTN_EINVAL and b"aligned" in lib.attn_last_error()
