"""fp64 CPU oracle for multi-head scaled-dot-product self-attention.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark import this module to check the HIP library.  The library
and its Python binding never import it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
independent rows); this module only builds it with gcc, checks shapes and
marshals numpy arrays.  See ``oracle.c`` for the definition followed and the
pages it cites (llm.c ``attention_backward.cu`` CPU references and the
self-attention formula of "Umakini wa kujitegemea, kerneli za CUDA na
FlashAttention", section 1).

Every function here is pinned by ``tests/test_oracle.py`` (rows summing to 1,
exact zeros under the mask, T=1, closed forms for uniform attention,
invariances, a hand-derived golden case, torch's fp64 attention, and central
finite differences for the backward).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            i = ctypes.c_int
            lib.oracle_forward.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i]
            lib.oracle_forward.restype = i
            lib.oracle_backward.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i]
            lib.oracle_backward.restype = i
            lib.oracle_forward_block.argtypes = [dp, dp, dp] + [i] * 9
            lib.oracle_forward_block.restype = i
            lib.oracle_layernorm_forward.argtypes = [dp] * 6 + [i, i]
            lib.oracle_layernorm_forward.restype = i
            lib.oracle_layernorm_backward.argtypes = [dp] * 6 + [i, i]
            lib.oracle_layernorm_backward.restype = i
            lib.oracle_set_threads.argtypes = [i]
            lib.oracle_set_threads.restype = None
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = i
            _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as_f64(x) -> np.ndarray:
    """Accept a numpy array or a CPU torch tensor; return contiguous float64."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _dims(qkv: np.ndarray, NH: int):
    if qkv.ndim != 3 or qkv.shape[2] % 3 != 0:
        raise ValueError(f"qkv must be (B, T, 3C), got {qkv.shape}")
    B, T, C3 = qkv.shape
    C = C3 // 3
    if NH < 1 or C % NH != 0:
        raise ValueError(f"C={C} is not a multiple of NH={NH}")
    return B, T, C


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def forward(qkv, NH: int, causal: bool = True, materialized: bool = False):
    """Return (out (B,T,C), lse (B,NH,T)) and, if materialized, also
    (preatt, att) of shape (B,NH,T,T), all float64."""
    qkv = _as_f64(qkv)
    B, T, C = _dims(qkv, NH)
    out = np.empty((B, T, C), np.float64)
    lse = np.empty((B, NH, T), np.float64)
    pre = np.empty((B, NH, T, T), np.float64) if materialized else None
    att = np.empty((B, NH, T, T), np.float64) if materialized else None
    rc = _load().oracle_forward(_ptr(out), _ptr(lse), _ptr(pre), _ptr(att), _ptr(qkv),
                                B, T, C, NH, int(bool(causal)))
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed with status {rc}")
    if materialized:
        return out, lse, pre, att
    return out, lse


def forward_block(qkv, NH: int, causal: bool, q0: int, q1: int, k0: int, k1: int):
    """Forward of query rows [q0, q1) against keys [k0, k1) (each row keeps
    its causal limit).  Return (out (B, q1-q0, C), lse (B, NH, q1-q0)),
    float64; rows with no key in the range get out 0 and lse -inf."""
    qkv = _as_f64(qkv)
    B, T, C = _dims(qkv, NH)
    nq = q1 - q0
    if not (0 <= q0 < q1 <= T and 0 <= k0 <= k1 <= T):
        raise ValueError(f"bad ranges q[{q0},{q1}) k[{k0},{k1}) for T={T}")
    out = np.empty((B, nq, C), np.float64)
    lse = np.empty((B, NH, nq), np.float64)
    rc = _load().oracle_forward_block(_ptr(out), _ptr(lse), _ptr(qkv), B, T, C, NH,
                                      int(bool(causal)), q0, q1, k0, k1)
    if rc != 0:
        raise RuntimeError(f"oracle_forward_block failed with status {rc}")
    return out, lse


def backward(qkv, dout, NH: int, causal: bool = True, materialized: bool = False):
    """Return dqkv (B,T,3C) and, if materialized, also (dpreatt, datt) of
    shape (B,NH,T,T), all float64."""
    qkv = _as_f64(qkv)
    dout = _as_f64(dout)
    B, T, C = _dims(qkv, NH)
    if dout.shape != (B, T, C):
        raise ValueError(f"dout must be {(B, T, C)}, got {dout.shape}")
    dqkv = np.empty((B, T, 3 * C), np.float64)
    dpre = np.empty((B, NH, T, T), np.float64) if materialized else None
    datt = np.empty((B, NH, T, T), np.float64) if materialized else None
    rc = _load().oracle_backward(_ptr(dqkv), _ptr(dpre), _ptr(datt), _ptr(dout), _ptr(qkv),
                                 B, T, C, NH, int(bool(causal)))
    if rc != 0:
        raise RuntimeError(f"oracle_backward failed with status {rc}")
    if materialized:
        return dqkv, dpre, datt
    return dqkv


def head_slice(x, b: int, h: int, NH: int, packed: bool):
    """Cut head (b, h) out of a packed qkv (B,T,3C) or an out-like (B,T,C)
    tensor, as a B=1, NH=1 tensor.  Heads are independent (section 1 of the
    self-attention page), so the oracle on the slice is the oracle of that
    head.  Pure indexing, no arithmetic."""
    x = _as_f64(x)
    if packed:
        C = x.shape[2] // 3
        hs = C // NH
        parts = [x[b:b + 1, :, p * C + h * hs: p * C + (h + 1) * hs] for p in range(3)]
        return np.ascontiguousarray(np.concatenate(parts, axis=2))
    C = x.shape[2]
    hs = C // NH
    return np.ascontiguousarray(x[b:b + 1, :, h * hs:(h + 1) * hs])


def layernorm_forward(inp, weight, bias):
    """LayerNorm of each row of inp (N, C) (oracle.c, layernorm part):
    return (out (N, C), mean (N,), rstd (N,)), float64, eps 1e-5."""
    x = _as_f64(inp)
    if x.ndim != 2:
        raise ValueError(f"inp must be (N, C), got {x.shape}")
    N, C = x.shape
    w, b = _as_f64(weight), _as_f64(bias)
    if w.shape != (C,) or b.shape != (C,):
        raise ValueError(f"weight and bias must be ({C},)")
    out = np.empty((N, C), np.float64)
    mean = np.empty((N,), np.float64)
    rstd = np.empty((N,), np.float64)
    rc = _load().oracle_layernorm_forward(_ptr(out), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(w),
                                          _ptr(b), N, C)
    if rc != 0:
        raise RuntimeError(f"oracle_layernorm_forward failed with status {rc}")
    return out, mean, rstd


def layernorm_backward(dout, inp, weight):
    """Gradients of the LayerNorm of inp (N, C) given dout (N, C): return
    (dinp (N, C), dweight (C,), dbias (C,)), float64."""
    x, dy, w = _as_f64(inp), _as_f64(dout), _as_f64(weight)
    if x.ndim != 2 or dy.shape != x.shape:
        raise ValueError(f"inp and dout must both be (N, C), got {x.shape} and {dy.shape}")
    N, C = x.shape
    if w.shape != (C,):
        raise ValueError(f"weight must be ({C},)")
    dx = np.empty((N, C), np.float64)
    dw = np.empty((C,), np.float64)
    db = np.empty((C,), np.float64)
    rc = _load().oracle_layernorm_backward(_ptr(dx), _ptr(dw), _ptr(db), _ptr(dy), _ptr(x),
                                           _ptr(w), N, C)
    if rc != 0:
        raise RuntimeError(f"oracle_layernorm_backward failed with status {rc}")
    return dx, dw, db
