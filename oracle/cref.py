"""ctypes binding of oracle/layer_ref.c: the oracle's layer step as plain threaded C loops in fp64.

TEST INFRASTRUCTURE ONLY (the CPU baseline's form of the oracle; the tests pin it against the
brute-force and numpy forms). build() compiles it with the host C compiler; nothing on the
product path loads it.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "layer_ref.c")
LIB = os.path.join(HERE, "_lib", "liboracle_ref.so")
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
_lib = None


def build() -> str:
    """Compile layer_ref.c into oracle/_lib/liboracle_ref.so (-O2, no fast-math: IEEE fp64)."""
    cc = os.environ.get("CC") or shutil.which("gcc") or "cc"
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math", SRC, "-o", tmp, "-lm"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"oracle C build failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        I = ctypes.c_int
        L.oref_layer_step.argtypes = [f32p, f32p, f32p, f32p, f32p, f32p, i32p, I, I, I, I, I, I, I, I, i32p, I,
                                      ctypes.POINTER(ctypes.c_double), I]
        L.oref_layer_step.restype = I
        L.oref_round.argtypes = [ctypes.c_double, I]
        L.oref_round.restype = ctypes.c_double
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def round_to_dtype(x: float, dtype: str) -> float:
    return lib().oref_round(float(x), DTYPES[dtype])


def _f32(a, name):
    a = np.asarray(a)
    if a.dtype != np.float32 or not a.flags.c_contiguous:
        raise ValueError(f"{name} must be a C-contiguous float32 array")
    return a


def layer_step(x, wq, wk, wv, kc, vc, past_len, n_q_heads: int, dtype: str, t_index=None, threads=None):
    """oracle.layer_step (without the rotary embedding) in C: appends the new K/V rows to kc, vc
    (float32 [B, Hkv, cap, d], modified in place) and returns O [B, n, Hq, d] in fp64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wq = np.ascontiguousarray(wq, dtype=np.float32)
    wk = np.ascontiguousarray(wk, dtype=np.float32)
    wv = np.ascontiguousarray(wv, dtype=np.float32)
    kc, vc = _f32(kc, "kc"), _f32(vc, "vc")
    B, T, D = x.shape
    Hkv, cap, d = kc.shape[1], kc.shape[2], kc.shape[3]
    if kc.shape != vc.shape or kc.shape[0] != B:
        raise ValueError("kc and vc must both be [B, Hkv, cap, d]")
    if wq.shape != (D, n_q_heads * d) or wk.shape != (D, Hkv * d) or wv.shape != (D, Hkv * d):
        raise ValueError("weights must be wq [D, Hq*d], wk and wv [D, Hkv*d]")
    ts = np.arange(T, dtype=np.int32) if t_index is None else np.ascontiguousarray(t_index, dtype=np.int32)
    lens = np.ascontiguousarray(past_len, dtype=np.int32)
    out = np.zeros((B, len(ts), n_q_heads, d), dtype=np.float64)
    f32p = ctypes.POINTER(ctypes.c_float)
    i32p = ctypes.POINTER(ctypes.c_int32)
    st = lib().oref_layer_step(
        x.ctypes.data_as(f32p), wq.ctypes.data_as(f32p), wk.ctypes.data_as(f32p), wv.ctypes.data_as(f32p),
        kc.ctypes.data_as(f32p), vc.ctypes.data_as(f32p), lens.ctypes.data_as(i32p), B, T, D, n_q_heads, Hkv, d,
        cap, DTYPES[dtype], ts.ctypes.data_as(i32p), len(ts), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        int(threads or default_threads()))
    if st != 0:
        raise ValueError("oracle C layer step refused its arguments (shapes, lengths past capacity, or memory)")
    return out
