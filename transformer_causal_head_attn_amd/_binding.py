"""ctypes binding of libattn's C ABI (argument marshalling only).

Every function named like an entry point of ``include/libattn.h`` takes torch
tensors where the C call takes device pointers, checks that they are
contiguous CUDA (HIP) tensors of the right dtype and size, passes
``data_ptr()`` and torch's current stream, and raises ``AttnError`` on a
non-zero status.  All arithmetic runs in the HIP kernels of libattn.so; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_EHIP = -3

EXPORTS = (
    "attn_forward", "attn_backward", "attn_backward_noalloc",
    "attn_backward_prepare", "attn_backward_dkdvdq",
    "attn_backward_preprocess", "attn_backward_dkdv", "attn_backward_dq",
    "attn_backward_ds_bytes", "attn_backward_dkdv_ds", "attn_backward_dq_ds",
    "attn_forward_bf16", "attn_backward_bf16",
    "attn_backward_preprocess_bf16", "attn_backward_dkdv_bf16", "attn_backward_dq_bf16",
    "attn_forward_f16", "attn_backward_f16", "attn_forward_fp8",
    "attn_forward_splitkv_chunk", "attn_forward_splitkv_bytes",
    "attn_forward_splitkv_bf16", "attn_forward_splitkv_f16",
    "attn_backward_splitkv_bytes", "attn_backward_splitkv_bf16", "attn_backward_splitkv_f16",
    "attn_backward_preprocess_f16", "attn_backward_dkdv_f16", "attn_backward_dq_f16",
    "attn_forward_materialized", "attn_backward_materialized",
    "attn_decode", "attn_decode_bf16", "attn_decode_f16",
    "attn_merge", "attn_merge_bf16", "attn_merge_f16",
    "layernorm_forward", "layernorm_forward_bf16", "layernorm_backward", "layernorm_backward_bf16",
    "layernorm_forward_f16", "layernorm_backward_f16",
    "attn_qkv_projection", "attn_qkv_projection_bf16",
    "attn_out_projection", "attn_out_projection_bf16",
    "attn_set_stream", "attn_last_error", "attn_release",
)


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


_lock = threading.Lock()
_lib = None


def load(path: str | None = None):
    """Load libattn.so (building it first only if it does not exist)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(p)
        vp, i = ctypes.c_void_p, ctypes.c_int
        for name, nptr in (("attn_forward", 3), ("attn_forward_bf16", 3),
                           ("attn_backward", 5), ("attn_backward_bf16", 5),
                           ("attn_backward_noalloc", 5),
                           ("attn_forward_materialized", 4),
                           ("attn_backward_materialized", 6),
                           ("attn_backward_dkdv", 5), ("attn_backward_dq", 6),
                           ("attn_backward_dkdvdq", 5),
                           ("attn_backward_dkdv_bf16", 5), ("attn_backward_dq_bf16", 6),
                           ("attn_forward_f16", 3), ("attn_backward_f16", 5),
                           ("attn_forward_fp8", 3),
                           ("attn_backward_dkdv_f16", 5), ("attn_backward_dq_f16", 6)):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * nptr + [i] * 5
            fn.restype = i
        for name in ("attn_backward_preprocess", "attn_backward_preprocess_bf16",
                     "attn_backward_preprocess_f16",
                     "attn_decode", "attn_decode_bf16", "attn_decode_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 3 + [i] * 4
            fn.restype = i
        lib.attn_backward_prepare.argtypes = [vp] * 4 + [i] * 4
        lib.attn_backward_prepare.restype = i
        lib.attn_forward_splitkv_chunk.argtypes = [i] * 5
        lib.attn_forward_splitkv_chunk.restype = i
        lib.attn_forward_splitkv_bytes.argtypes = [i] * 6
        lib.attn_forward_splitkv_bytes.restype = ctypes.c_uint64
        for name in ("attn_forward_splitkv_bf16", "attn_forward_splitkv_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 4 + [i] * 6
            fn.restype = i
        lib.attn_backward_splitkv_bytes.argtypes = [i] * 6
        lib.attn_backward_splitkv_bytes.restype = ctypes.c_uint64
        for name in ("attn_backward_splitkv_bf16", "attn_backward_splitkv_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 6 + [i] * 6
            fn.restype = i
        lib.attn_backward_ds_bytes.argtypes = [i] * 5
        lib.attn_backward_ds_bytes.restype = ctypes.c_uint64
        lib.attn_backward_dkdv_ds.argtypes = [vp] * 6 + [i] * 5
        lib.attn_backward_dkdv_ds.restype = i
        lib.attn_backward_dq_ds.argtypes = [vp] * 3 + [i] * 5
        lib.attn_backward_dq_ds.restype = i
        for name in ("attn_merge", "attn_merge_bf16", "attn_merge_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 4 + [i] * 5
            fn.restype = i
        for name in ("layernorm_forward", "layernorm_forward_bf16", "layernorm_forward_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 6 + [i] * 2
            fn.restype = i
        for name in ("layernorm_backward", "layernorm_backward_bf16", "layernorm_backward_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 8 + [i] * 2
            fn.restype = i
        for name in ("attn_qkv_projection", "attn_qkv_projection_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 4 + [i] * 3
            fn.restype = i
        for name in ("attn_out_projection", "attn_out_projection_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp] * 5 + [i] * 3
            fn.restype = i
        lib.attn_set_stream.argtypes = [vp]
        lib.attn_set_stream.restype = i
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_release.argtypes = []
        lib.attn_release.restype = None
        _lib = lib
        return lib


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, numel: int) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _call(name: str, *args) -> None:
    lib = load()
    lib.attn_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    rc = getattr(lib, name)(*args)
    if rc != ATTN_OK:
        raise AttnError(name, rc, lib.attn_last_error().decode())


def _dims(B, T, C, NH, causal):
    return [int(B), int(T), int(C), int(NH), int(causal)]


# ------------------------------------------------------- C ABI, one to one --

def attn_forward(out, lse, qkv, B, T, C, NH, causal) -> None:
    f = torch.float32
    _call("attn_forward", _check(out, "out", f, B * T * C), _check(lse, "lse", f, B * NH * T),
          _check(qkv, "qkv", f, B * T * 3 * C), *_dims(B, T, C, NH, causal))


def attn_backward(dqkv, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    f = torch.float32
    _call("attn_backward", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(dout, "dout", f, B * T * C), _check(qkv, "qkv", f, B * T * 3 * C),
          _check(out, "out", f, B * T * C), _check(lse, "lse", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_noalloc(dqkv, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    f = torch.float32
    _call("attn_backward_noalloc", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(dout, "dout", f, B * T * C), _check(qkv, "qkv", f, B * T * 3 * C),
          _check(out, "out", f, B * T * C), _check(lse, "lse", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_prepare(dqkv, D, dout, out, B, T, C, NH) -> None:
    f = torch.float32
    _call("attn_backward_prepare", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(D, "D", f, B * NH * T), _check(dout, "dout", f, B * T * C),
          _check(out, "out", f, B * T * C), int(B), int(T), int(C), int(NH))


def attn_backward_dkdvdq(dqkv, dout, qkv, lse, D, B, T, C, NH, causal) -> None:
    f = torch.float32
    _call("attn_backward_dkdvdq", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(dout, "dout", f, B * T * C), _check(qkv, "qkv", f, B * T * 3 * C),
          _check(lse, "lse", f, B * NH * T), _check(D, "D", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_preprocess(D, dout, out, B, T, C, NH) -> None:
    f = torch.float32
    _call("attn_backward_preprocess", _check(D, "D", f, B * NH * T),
          _check(dout, "dout", f, B * T * C), _check(out, "out", f, B * T * C),
          int(B), int(T), int(C), int(NH))


def attn_backward_dkdv(dqkv, dout, qkv, lse, D, B, T, C, NH, causal) -> None:
    f = torch.float32
    _call("attn_backward_dkdv", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(dout, "dout", f, B * T * C), _check(qkv, "qkv", f, B * T * 3 * C),
          _check(lse, "lse", f, B * NH * T), _check(D, "D", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_dq(dqkv, D, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    f = torch.float32
    _call("attn_backward_dq", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(D, "D", f, B * NH * T), _check(dout, "dout", f, B * T * C),
          _check(qkv, "qkv", f, B * T * 3 * C), _check(out, "out", f, B * T * C),
          _check(lse, "lse", f, B * NH * T), *_dims(B, T, C, NH, causal))


def attn_forward_splitkv_chunk(B, T, C, NH, causal) -> int:
    """Keys per chunk the split-KV forward picks for this shape (raises on
    invalid arguments)."""
    lib = load()
    rc = lib.attn_forward_splitkv_chunk(*_dims(B, T, C, NH, causal))
    if rc < 0:
        raise AttnError("attn_forward_splitkv_chunk", rc, lib.attn_last_error().decode())
    return int(rc)


def attn_forward_splitkv_bytes(B, T, C, NH, causal, kv_chunk) -> int:
    """Bytes of the split-KV forward's work buffer (0: no split, or invalid
    arguments)."""
    return int(load().attn_forward_splitkv_bytes(*_dims(B, T, C, NH, causal), int(kv_chunk)))


def _splitkv(name, dtype, out, lse, qkv, work, B, T, C, NH, causal, kv_chunk):
    nw = attn_forward_splitkv_bytes(B, T, C, NH, causal, kv_chunk) // 4
    if work.numel() < nw:
        raise ValueError(f"work has {work.numel()} floats, the split needs {nw}")
    _call(name, _check(out, "out", dtype, B * T * C), _check(lse, "lse", torch.float32, B * NH * T),
          _check(qkv, "qkv", dtype, B * T * 3 * C),
          _check(work, "work", torch.float32, work.numel()),
          *_dims(B, T, C, NH, causal), int(kv_chunk))


def attn_forward_splitkv_bf16(out, lse, qkv, work, B, T, C, NH, causal, kv_chunk) -> None:
    _splitkv("attn_forward_splitkv_bf16", torch.bfloat16, out, lse, qkv, work, B, T, C, NH, causal,
             kv_chunk)


def attn_forward_splitkv_f16(out, lse, qkv, work, B, T, C, NH, causal, kv_chunk) -> None:
    _splitkv("attn_forward_splitkv_f16", torch.float16, out, lse, qkv, work, B, T, C, NH, causal,
             kv_chunk)


def attn_backward_splitkv_bytes(B, T, C, NH, causal, kv_chunk) -> int:
    """Bytes of the split backward's work buffer (0 for invalid arguments)."""
    return int(load().attn_backward_splitkv_bytes(*_dims(B, T, C, NH, causal), int(kv_chunk)))


def _bwd_splitkv(name, dtype, dqkv, dout, qkv, out, lse, work, B, T, C, NH, causal, kv_chunk):
    nw = attn_backward_splitkv_bytes(B, T, C, NH, causal, kv_chunk) // 4
    if work.numel() < nw:
        raise ValueError(f"work has {work.numel()} floats, the split needs {nw}")
    _call(name, _check(dqkv, "dqkv", dtype, B * T * 3 * C), _check(dout, "dout", dtype, B * T * C),
          _check(qkv, "qkv", dtype, B * T * 3 * C), _check(out, "out", dtype, B * T * C),
          _check(lse, "lse", torch.float32, B * NH * T),
          _check(work, "work", torch.float32, work.numel()),
          *_dims(B, T, C, NH, causal), int(kv_chunk))


def attn_backward_splitkv_bf16(dqkv, dout, qkv, out, lse, work, B, T, C, NH, causal,
                               kv_chunk) -> None:
    _bwd_splitkv("attn_backward_splitkv_bf16", torch.bfloat16, dqkv, dout, qkv, out, lse, work,
                 B, T, C, NH, causal, kv_chunk)


def attn_backward_splitkv_f16(dqkv, dout, qkv, out, lse, work, B, T, C, NH, causal,
                              kv_chunk) -> None:
    _bwd_splitkv("attn_backward_splitkv_f16", torch.float16, dqkv, dout, qkv, out, lse, work,
                 B, T, C, NH, causal, kv_chunk)


def attn_qkv_projection(qkv, x, w, bias, M, K, N) -> None:
    f = torch.float32
    _call("attn_qkv_projection", _check(qkv, "qkv", f, M * N), _check(x, "x", f, M * K),
          _check(w, "w", f, N * K), _check(bias, "bias", f, N), int(M), int(K), int(N))


def attn_qkv_projection_bf16(qkv, x, w, bias, M, K, N) -> None:
    h = torch.bfloat16
    _call("attn_qkv_projection_bf16", _check(qkv, "qkv", h, M * N), _check(x, "x", h, M * K),
          _check(w, "w", h, N * K), _check(bias, "bias", torch.float32, N),
          int(M), int(K), int(N))


def attn_out_projection(y, a, w, bias, residual, M, K, N) -> None:
    f = torch.float32
    _call("attn_out_projection", _check(y, "y", f, M * N), _check(a, "a", f, M * K),
          _check(w, "w", f, N * K), _check(bias, "bias", f, N),
          _check(residual, "residual", f, M * N), int(M), int(K), int(N))


def attn_out_projection_bf16(y, a, w, bias, residual, M, K, N) -> None:
    h = torch.bfloat16
    _call("attn_out_projection_bf16", _check(y, "y", h, M * N), _check(a, "a", h, M * K),
          _check(w, "w", h, N * K), _check(bias, "bias", torch.float32, N),
          _check(residual, "residual", h, M * N), int(M), int(K), int(N))


def qkv_projection(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    """Allocate qkv with torch and run x w^T + bias (x (..., K), w (N, K));
    fp32 or bf16 by x's dtype, bias fp32."""
    K = x.shape[-1]
    M = x.numel() // K
    N = w.shape[0]
    out = torch.empty(x.shape[:-1] + (N,), dtype=x.dtype, device=x.device)
    fn = attn_qkv_projection_bf16 if x.dtype == torch.bfloat16 else attn_qkv_projection
    fn(out, x, w, bias, M, K, N)
    return out


def out_projection(a: torch.Tensor, w: torch.Tensor, bias: torch.Tensor,
                   residual: torch.Tensor) -> torch.Tensor:
    """Allocate y with torch and run a w^T + bias + residual."""
    K = a.shape[-1]
    M = a.numel() // K
    N = w.shape[0]
    out = torch.empty(a.shape[:-1] + (N,), dtype=a.dtype, device=a.device)
    fn = attn_out_projection_bf16 if a.dtype == torch.bfloat16 else attn_out_projection
    fn(out, a, w, bias, residual, M, K, N)
    return out


def attn_backward_ds_bytes(B, T, C, NH, causal) -> int:
    """Bytes of the dS block store for this shape (0 for invalid arguments)."""
    return int(load().attn_backward_ds_bytes(*_dims(B, T, C, NH, causal)))


def attn_backward_dkdv_ds(dqkv, dS, dout, qkv, lse, D, B, T, C, NH, causal) -> None:
    f = torch.float32
    nds = attn_backward_ds_bytes(B, T, C, NH, causal) // 4
    _call("attn_backward_dkdv_ds", _check(dqkv, "dqkv", f, B * T * 3 * C), _check(dS, "dS", f, nds),
          _check(dout, "dout", f, B * T * C), _check(qkv, "qkv", f, B * T * 3 * C),
          _check(lse, "lse", f, B * NH * T), _check(D, "D", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_dq_ds(dqkv, dS, qkv, B, T, C, NH, causal) -> None:
    f = torch.float32
    nds = attn_backward_ds_bytes(B, T, C, NH, causal) // 4
    _call("attn_backward_dq_ds", _check(dqkv, "dqkv", f, B * T * 3 * C), _check(dS, "dS", f, nds),
          _check(qkv, "qkv", f, B * T * 3 * C), *_dims(B, T, C, NH, causal))


def attn_forward_bf16(out, lse, qkv, B, T, C, NH, causal) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_forward_bf16", _check(out, "out", h, B * T * C), _check(lse, "lse", f, B * NH * T),
          _check(qkv, "qkv", h, B * T * 3 * C), *_dims(B, T, C, NH, causal))


def attn_forward_fp8(out, lse, qkv, B, T, C, NH, causal) -> None:
    """qkv: torch.float8_e4m3fn (OCP E4M3); out: bfloat16; lse: float32."""
    _call("attn_forward_fp8", _check(out, "out", torch.bfloat16, B * T * C),
          _check(lse, "lse", torch.float32, B * NH * T),
          _check(qkv, "qkv", torch.float8_e4m3fn, B * T * 3 * C), *_dims(B, T, C, NH, causal))


def forward_fp8(qkv: torch.Tensor, NH: int, causal: bool = True):
    """Allocate (out bf16, lse fp32) with torch and run the fp8 forward on a
    float8_e4m3fn qkv."""
    B, T, C = _shape(qkv, NH)
    out = torch.empty((B, T, C), dtype=torch.bfloat16, device=qkv.device)
    lse = torch.empty((B, NH, T), dtype=torch.float32, device=qkv.device)
    attn_forward_fp8(out, lse, qkv, B, T, C, NH, int(causal))
    return out, lse


def attn_backward_bf16(dqkv, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_backward_bf16", _check(dqkv, "dqkv", h, B * T * 3 * C),
          _check(dout, "dout", h, B * T * C), _check(qkv, "qkv", h, B * T * 3 * C),
          _check(out, "out", h, B * T * C), _check(lse, "lse", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_preprocess_bf16(D, dout, out, B, T, C, NH) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_backward_preprocess_bf16", _check(D, "D", f, B * NH * T),
          _check(dout, "dout", h, B * T * C), _check(out, "out", h, B * T * C),
          int(B), int(T), int(C), int(NH))


def attn_backward_dkdv_bf16(dqkv, dout, qkv, lse, D, B, T, C, NH, causal) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_backward_dkdv_bf16", _check(dqkv, "dqkv", h, B * T * 3 * C),
          _check(dout, "dout", h, B * T * C), _check(qkv, "qkv", h, B * T * 3 * C),
          _check(lse, "lse", f, B * NH * T), _check(D, "D", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_dq_bf16(dqkv, D, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_backward_dq_bf16", _check(dqkv, "dqkv", h, B * T * 3 * C),
          _check(D, "D", f, B * NH * T), _check(dout, "dout", h, B * T * C),
          _check(qkv, "qkv", h, B * T * 3 * C), _check(out, "out", h, B * T * C),
          _check(lse, "lse", f, B * NH * T), *_dims(B, T, C, NH, causal))


def attn_forward_f16(out, lse, qkv, B, T, C, NH, causal) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_forward_f16", _check(out, "out", h, B * T * C), _check(lse, "lse", f, B * NH * T),
          _check(qkv, "qkv", h, B * T * 3 * C), *_dims(B, T, C, NH, causal))


def attn_backward_f16(dqkv, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_backward_f16", _check(dqkv, "dqkv", h, B * T * 3 * C),
          _check(dout, "dout", h, B * T * C), _check(qkv, "qkv", h, B * T * 3 * C),
          _check(out, "out", h, B * T * C), _check(lse, "lse", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_preprocess_f16(D, dout, out, B, T, C, NH) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_backward_preprocess_f16", _check(D, "D", f, B * NH * T),
          _check(dout, "dout", h, B * T * C), _check(out, "out", h, B * T * C),
          int(B), int(T), int(C), int(NH))


def attn_backward_dkdv_f16(dqkv, dout, qkv, lse, D, B, T, C, NH, causal) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_backward_dkdv_f16", _check(dqkv, "dqkv", h, B * T * 3 * C),
          _check(dout, "dout", h, B * T * C), _check(qkv, "qkv", h, B * T * 3 * C),
          _check(lse, "lse", f, B * NH * T), _check(D, "D", f, B * NH * T),
          *_dims(B, T, C, NH, causal))


def attn_backward_dq_f16(dqkv, D, dout, qkv, out, lse, B, T, C, NH, causal) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_backward_dq_f16", _check(dqkv, "dqkv", h, B * T * 3 * C),
          _check(D, "D", f, B * NH * T), _check(dout, "dout", h, B * T * C),
          _check(qkv, "qkv", h, B * T * 3 * C), _check(out, "out", h, B * T * C),
          _check(lse, "lse", f, B * NH * T), *_dims(B, T, C, NH, causal))


def attn_forward_materialized(out, preatt, att, qkv, B, T, C, NH, causal) -> None:
    f = torch.float32
    M = B * NH * T * T
    _call("attn_forward_materialized", _check(out, "out", f, B * T * C),
          _check(preatt, "preatt", f, M), _check(att, "att", f, M),
          _check(qkv, "qkv", f, B * T * 3 * C), *_dims(B, T, C, NH, causal))


def attn_backward_materialized(dqkv, dpreatt, datt, dout, qkv, att, B, T, C, NH, causal) -> None:
    f = torch.float32
    M = B * NH * T * T
    _call("attn_backward_materialized", _check(dqkv, "dqkv", f, B * T * 3 * C),
          _check(dpreatt, "dpreatt", f, M), _check(datt, "datt", f, M),
          _check(dout, "dout", f, B * T * C), _check(qkv, "qkv", f, B * T * 3 * C),
          _check(att, "att", f, M), *_dims(B, T, C, NH, causal))


def attn_decode(out, lse, qkv, B, T, C, NH) -> None:
    f = torch.float32
    _call("attn_decode", _check(out, "out", f, B * C), _check(lse, "lse", f, B * NH),
          _check(qkv, "qkv", f, B * T * 3 * C), int(B), int(T), int(C), int(NH))


def attn_decode_bf16(out, lse, qkv, B, T, C, NH) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_decode_bf16", _check(out, "out", h, B * C), _check(lse, "lse", f, B * NH),
          _check(qkv, "qkv", h, B * T * 3 * C), int(B), int(T), int(C), int(NH))


def attn_decode_f16(out, lse, qkv, B, T, C, NH) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_decode_f16", _check(out, "out", h, B * C), _check(lse, "lse", f, B * NH),
          _check(qkv, "qkv", h, B * T * 3 * C), int(B), int(T), int(C), int(NH))


def attn_merge(out, lse, o_parts, lse_parts, nparts, B, T, C, NH) -> None:
    f = torch.float32
    _call("attn_merge", _check(out, "out", f, B * T * C), _check(lse, "lse", f, B * NH * T),
          _check(o_parts, "o_parts", f, nparts * B * T * C),
          _check(lse_parts, "lse_parts", f, nparts * B * NH * T),
          int(nparts), int(B), int(T), int(C), int(NH))


def attn_merge_bf16(out, lse, o_parts, lse_parts, nparts, B, T, C, NH) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("attn_merge_bf16", _check(out, "out", h, B * T * C), _check(lse, "lse", f, B * NH * T),
          _check(o_parts, "o_parts", f, nparts * B * T * C),
          _check(lse_parts, "lse_parts", f, nparts * B * NH * T),
          int(nparts), int(B), int(T), int(C), int(NH))


def attn_merge_f16(out, lse, o_parts, lse_parts, nparts, B, T, C, NH) -> None:
    h, f = torch.float16, torch.float32
    _call("attn_merge_f16", _check(out, "out", h, B * T * C), _check(lse, "lse", f, B * NH * T),
          _check(o_parts, "o_parts", f, nparts * B * T * C),
          _check(lse_parts, "lse_parts", f, nparts * B * NH * T),
          int(nparts), int(B), int(T), int(C), int(NH))


def attn_set_stream(stream) -> None:
    """Set the calling thread's libattn stream (a torch.cuda.Stream, a raw
    hipStream_t integer, or None for the null stream).  The functions above
    set torch's current stream before every call anyway."""
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    load().attn_set_stream(ctypes.c_void_p(stream or 0))


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def attn_release() -> None:
    load().attn_release()


# ---------------------------------------------------- allocating helpers --

def _shape(qkv: torch.Tensor, NH: int):
    if qkv.dim() != 3 or qkv.shape[2] % 3:
        raise ValueError(f"qkv must be (B, T, 3C), got {tuple(qkv.shape)}")
    B, T, C3 = qkv.shape
    return B, T, C3 // 3


def forward(qkv: torch.Tensor, NH: int, causal: bool = True):
    """Allocate (out, lse) with torch and run the fused forward (fp32, bf16
    or fp16 by qkv's dtype)."""
    B, T, C = _shape(qkv, NH)
    out = torch.empty((B, T, C), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, NH, T), dtype=torch.float32, device=qkv.device)
    fn = {torch.bfloat16: attn_forward_bf16, torch.float16: attn_forward_f16}.get(qkv.dtype, attn_forward)
    fn(out, lse, qkv, B, T, C, NH, int(causal))
    return out, lse


def forward_splitkv(qkv: torch.Tensor, NH: int, causal: bool = True, kv_chunk: int = 0):
    """Allocate (out, lse) and the work buffer with torch and run the split-KV
    forward (bf16 or fp16 by qkv's dtype)."""
    B, T, C = _shape(qkv, NH)
    out = torch.empty((B, T, C), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, NH, T), dtype=torch.float32, device=qkv.device)
    nw = attn_forward_splitkv_bytes(B, T, C, NH, int(causal), kv_chunk) // 4
    work = torch.empty((max(nw, 4),), dtype=torch.float32, device=qkv.device)
    fn = {torch.bfloat16: attn_forward_splitkv_bf16, torch.float16: attn_forward_splitkv_f16}[qkv.dtype]
    fn(out, lse, qkv, work, B, T, C, NH, int(causal), kv_chunk)
    return out, lse


def backward_splitkv(dout, qkv, out, lse, NH: int, causal: bool = True, kv_chunk: int = 0):
    """Allocate dqkv and the work buffer with torch and run the split
    backward (bf16 or fp16 by qkv's dtype)."""
    B, T, C = _shape(qkv, NH)
    dqkv = torch.empty_like(qkv)
    nw = attn_backward_splitkv_bytes(B, T, C, NH, int(causal), kv_chunk) // 4
    work = torch.empty((max(nw, 4),), dtype=torch.float32, device=qkv.device)
    fn = {torch.bfloat16: attn_backward_splitkv_bf16, torch.float16: attn_backward_splitkv_f16}[qkv.dtype]
    fn(dqkv, dout, qkv, out, lse, work, B, T, C, NH, int(causal), kv_chunk)
    return dqkv


def backward(dout, qkv, out, lse, NH: int, causal: bool = True):
    """Allocate dqkv with torch and run the fused backward."""
    B, T, C = _shape(qkv, NH)
    dqkv = torch.empty_like(qkv)
    fn = {torch.bfloat16: attn_backward_bf16, torch.float16: attn_backward_f16}.get(qkv.dtype, attn_backward)
    fn(dqkv, dout, qkv, out, lse, B, T, C, NH, int(causal))
    return dqkv


def forward_materialized(qkv: torch.Tensor, NH: int, causal: bool = True):
    B, T, C = _shape(qkv, NH)
    out = torch.empty((B, T, C), dtype=torch.float32, device=qkv.device)
    pre = torch.empty((B, NH, T, T), dtype=torch.float32, device=qkv.device)
    att = torch.empty_like(pre)
    attn_forward_materialized(out, pre, att, qkv, B, T, C, NH, int(causal))
    return out, pre, att


def backward_materialized(dout, qkv, att, NH: int, causal: bool = True):
    B, T, C = _shape(qkv, NH)
    dqkv = torch.empty_like(qkv)
    dpre = torch.empty_like(att)
    datt = torch.empty_like(att)
    attn_backward_materialized(dqkv, dpre, datt, dout, qkv, att, B, T, C, NH, int(causal))
    return dqkv, dpre, datt


def layernorm_forward(out, mean, rstd, inp, weight, bias, N, C) -> None:
    f = torch.float32
    _call("layernorm_forward", _check(out, "out", f, N * C), _check(mean, "mean", f, N),
          _check(rstd, "rstd", f, N), _check(inp, "inp", f, N * C),
          _check(weight, "weight", f, C), _check(bias, "bias", f, C), int(N), int(C))


def layernorm_forward_bf16(out, mean, rstd, inp, weight, bias, N, C) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("layernorm_forward_bf16", _check(out, "out", h, N * C), _check(mean, "mean", f, N),
          _check(rstd, "rstd", f, N), _check(inp, "inp", h, N * C),
          _check(weight, "weight", f, C), _check(bias, "bias", f, C), int(N), int(C))


def layernorm_backward(dinp, dweight, dbias, dout, inp, weight, mean, rstd, N, C) -> None:
    f = torch.float32
    _call("layernorm_backward", _check(dinp, "dinp", f, N * C), _check(dweight, "dweight", f, C),
          _check(dbias, "dbias", f, C), _check(dout, "dout", f, N * C),
          _check(inp, "inp", f, N * C), _check(weight, "weight", f, C),
          _check(mean, "mean", f, N), _check(rstd, "rstd", f, N), int(N), int(C))


def layernorm_backward_bf16(dinp, dweight, dbias, dout, inp, weight, mean, rstd, N, C) -> None:
    h, f = torch.bfloat16, torch.float32
    _call("layernorm_backward_bf16", _check(dinp, "dinp", h, N * C),
          _check(dweight, "dweight", f, C), _check(dbias, "dbias", f, C),
          _check(dout, "dout", h, N * C), _check(inp, "inp", h, N * C),
          _check(weight, "weight", f, C), _check(mean, "mean", f, N), _check(rstd, "rstd", f, N),
          int(N), int(C))


def layernorm_forward_f16(out, mean, rstd, inp, weight, bias, N, C) -> None:
    h, f = torch.float16, torch.float32
    _call("layernorm_forward_f16", _check(out, "out", h, N * C), _check(mean, "mean", f, N),
          _check(rstd, "rstd", f, N), _check(inp, "inp", h, N * C),
          _check(weight, "weight", f, C), _check(bias, "bias", f, C), int(N), int(C))


def layernorm_backward_f16(dinp, dweight, dbias, dout, inp, weight, mean, rstd, N, C) -> None:
    h, f = torch.float16, torch.float32
    _call("layernorm_backward_f16", _check(dinp, "dinp", h, N * C),
          _check(dweight, "dweight", f, C), _check(dbias, "dbias", f, C),
          _check(dout, "dout", h, N * C), _check(inp, "inp", h, N * C),
          _check(weight, "weight", f, C), _check(mean, "mean", f, N), _check(rstd, "rstd", f, N),
          int(N), int(C))


def layernorm(inp: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor):
    """Allocate and return (out, mean, rstd) for the LayerNorm of the rows
    of inp (..., C), fp32, bf16 or fp16 by inp's dtype."""
    C = inp.shape[-1]
    N = inp.numel() // C
    out = torch.empty_like(inp)
    mean = torch.empty(N, dtype=torch.float32, device=inp.device)
    rstd = torch.empty(N, dtype=torch.float32, device=inp.device)
    fn = {torch.bfloat16: layernorm_forward_bf16,
          torch.float16: layernorm_forward_f16}.get(inp.dtype, layernorm_forward)
    fn(out, mean, rstd, inp, weight, bias, N, C)
    return out, mean, rstd


def layernorm_grad(dout, inp, weight, mean, rstd):
    """Allocate and return (dinp, dweight, dbias) of the LayerNorm."""
    C = inp.shape[-1]
    N = inp.numel() // C
    dinp = torch.empty_like(inp)
    dw = torch.empty(C, dtype=torch.float32, device=inp.device)
    db = torch.empty(C, dtype=torch.float32, device=inp.device)
    fn = {torch.bfloat16: layernorm_backward_bf16,
          torch.float16: layernorm_backward_f16}.get(inp.dtype, layernorm_backward)
    fn(dinp, dw, db, dout, inp, weight, mean, rstd, N, C)
    return dinp, dw, db


def decode(qkv: torch.Tensor, NH: int):
    """Allocate (out (B, C), lse (B, NH)) and run the decode for the last
    position of each sequence (fp32, bf16 or fp16 by qkv's dtype)."""
    B, T, C = _shape(qkv, NH)
    out = torch.empty((B, C), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, NH), dtype=torch.float32, device=qkv.device)
    fn = {torch.bfloat16: attn_decode_bf16, torch.float16: attn_decode_f16}.get(qkv.dtype, attn_decode)
    fn(out, lse, qkv, B, T, C, NH)
    return out, lse


def merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out_dtype=torch.float32):
    """Merge partial results o_parts (P, B, T, C) fp32 and lse_parts
    (P, B, NH, T) into (out (B, T, C) of out_dtype, lse (B, NH, T))."""
    P, B, T, C = o_parts.shape
    NH = lse_parts.shape[2]
    out = torch.empty((B, T, C), dtype=out_dtype, device=o_parts.device)
    lse = torch.empty((B, NH, T), dtype=torch.float32, device=o_parts.device)
    fn = {torch.bfloat16: attn_merge_bf16, torch.float16: attn_merge_f16}.get(out_dtype, attn_merge)
    fn(out, lse, o_parts, lse_parts, P, B, T, C, NH)
    return out, lse
