"""Seeded synthetic inputs for one host-KV attention layer step.

This module draws random numbers and encodes them in the storage formats the layer uses
(fp32, IEEE fp16, bfloat16). It holds none of the layer's arithmetic: no projection,
no append, no softmax. Both the oracle-side tests and the GPU path take their inputs
from here, and from nowhere else, so that neither side generates data for the other.

Workloads are shaped after the pages' evaluation models: "Paper Notes: DirectKV",
section "Experiments & Results" (Llama-3.1-8B, 1K-32K contexts), and "DirectKV Guide",
section "Empirical Benchmarks" (Llama-3-70B at 64K-128K contexts). Values are synthetic:
X ~ N(0, 1), W ~ N(0, 1/D) (variance 1/D), past K/V ~ N(0, 1), all rounded to the
layer's dtype. No dataset or trained weight is involved.

Draw order for a named workload (numpy Generator(PCG64(seed))): Wq, Wk, Wv, the ragged
past lengths (if any), X of the first step, past K then past V (one (b, g) slice at a
time), then X of each later decode step.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def _bf16_round_f32(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Return float32 values exactly representable in `dtype` (input encoding only)."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a.copy()
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        return _bf16_round_f32(a)
    raise ValueError(dtype)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of dtype-exact float32 values: float32 for f32, uint16 otherwise."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return (a.view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def from_storage(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Inverse of `to_storage`: decode stored bit patterns to float32 (exact)."""
    if dtype == "f32":
        return np.asarray(bits).view(np.float32).astype(np.float32)
    if dtype == "f16":
        return np.asarray(bits).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


@dataclasses.dataclass
class Workload:
    """Shape of one layer step: B sequences, T new tokens each, past lengths `past`."""

    name: str
    dtype: str
    D: int
    Hq: int
    Hkv: int
    d: int
    B: int
    T: int
    past: Optional[List[int]]  # None: ragged, drawn from [past_lo, past_hi]
    cap: int
    past_lo: int = 0
    past_hi: int = 0
    decode_steps: int = 0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The workloads, in a fixed order; the seed of workload i is 1000 + i.
# cap = rows per (sequence, kv head) in the host cache, rounded up to a multiple of 64.
WORKLOADS = [
    Workload("tiny_f32_prefill128_decode1", "f32", D=256, Hq=4, Hkv=4, d=64,
             B=1, T=128, past=[0], cap=192, decode_steps=1, seed=1000),
    Workload("llama8b_decode_b8_L32768_bf16", "bf16", D=4096, Hq=32, Hkv=8, d=128,
             B=8, T=1, past=[32768] * 8, cap=32832, seed=1001),
    Workload("llama8b_prefill_T8192_on_L24576_bf16", "bf16", D=4096, Hq=32, Hkv=8, d=128,
             B=1, T=8192, past=[24576], cap=32768, seed=1002),
    Workload("long_decode_b4_L96k_128k_f16", "f16", D=4096, Hq=32, Hkv=8, d=128,
             B=4, T=1, past=None, cap=131136, past_lo=98304, past_hi=131072, seed=1003),
    Workload("llama70b_prefill_T16384_on_L49152_b2_bf16", "bf16", D=8192, Hq=64, Hkv=8, d=128,
             B=2, T=16384, past=[49152] * 2, cap=65600, decode_steps=64, seed=1004),
    # the other reading of the 70B-shaped case (a sensitivity row): the 65536 tokens are only
    # the cache capacity, the 16384-token prefill starts from an empty cache and the 64 decode
    # steps run at 16384 + s past tokens
    Workload("llama70b_prefill_T16384_empty_b2_bf16", "bf16", D=8192, Hq=64, Hkv=8, d=128,
             B=2, T=16384, past=[0] * 2, cap=16448, decode_steps=64, seed=1005),
]


def workload(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


class Draw:
    """Sequential draws for one layer step, in the documented order."""

    def __init__(self, seed: int):
        self.rng = np.random.Generator(np.random.PCG64(seed))

    def normal(self, shape, std: float, dtype: str) -> np.ndarray:
        a = self.rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a = a * np.float32(std)
        return quantize(a, dtype)

    def weights(self, D: int, ncols: int, dtype: str) -> np.ndarray:
        """W ~ N(0, 1/D), stored [D, ncols] and used as X @ W."""
        return self.normal((D, ncols), D ** -0.5, dtype)

    def lengths(self, B: int, lo: int, hi: int) -> np.ndarray:
        return self.rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)

    def integers(self, shape, lo: int, hi: int) -> np.ndarray:
        return self.rng.integers(lo, hi, size=shape, endpoint=True).astype(np.float32)


def layer_weights(draw: Draw, D: int, Hq: int, Hkv: int, d: int, dtype: str):
    wq = draw.weights(D, Hq * d, dtype)
    wk = draw.weights(D, Hkv * d, dtype)
    wv = draw.weights(D, Hkv * d, dtype)
    return wq, wk, wv


def stack_weights(draw: Draw, n_layers: int, D: int, Hq: int, Hkv: int, d: int, F: int, dtype: str):
    """Weights of a stack of pre-norm decoder layers, all stored [in, out] and used as X @ W,
    drawn layer by layer in this order: Wq, Wk, Wv [D, H·d] ~ N(0, 1/D); Wo [Hq·d, D] ~
    N(0, 1/(Hq·d)); the gate and up projections side by side, W_gu [D, 2F] ~ N(0, 1/D); W_down
    [F, D] ~ N(0, 1/F); the two norm weights g_attn, g_mlp [D] ~ 1 + N(0, 0.1^2)."""
    layers = []
    for _ in range(n_layers):
        wq, wk, wv = layer_weights(draw, D, Hq, Hkv, d, dtype)
        layers.append(dict(
            wq=wq, wk=wk, wv=wv,
            wo=draw.weights(Hq * d, D, dtype),
            w_gu=draw.weights(D, 2 * F, dtype),
            w_down=draw.weights(F, D, dtype),
            g_attn=quantize(1.0 + draw.normal((D,), 0.1, "f32"), dtype),
            g_mlp=quantize(1.0 + draw.normal((D,), 0.1, "f32"), dtype)))
    return layers


def fill_past(draw: Draw, kc: np.ndarray, vc: np.ndarray, past_len, dtype: str) -> None:
    """Write N(0, 1) past K (all slices) then past V into rows [0, past_len[b]) of
    caches shaped [B, Hkv, cap, d]. `kc`/`vc` may be float32 arrays or storage views."""
    B, Hkv = kc.shape[0], kc.shape[1]
    d = kc.shape[3]
    for cache in (kc, vc):
        for b in range(B):
            L = int(past_len[b])
            for g in range(Hkv):
                vals = draw.normal((L, d), 1.0, dtype)
                # float32 arrays take the values; uint16 storage views take bit patterns
                cache[b, g, :L, :] = vals if cache.dtype == np.float32 else to_storage(vals, dtype)


def sparse_sign_weights(draw: Draw, D: int, ncols: int, nnz: int = 8) -> np.ndarray:
    """Exact-arithmetic weights [D, ncols]: each column has `nnz` entries of +-1 at random
    rows and zeros elsewhere, so X·W with small-integer X is exact in every dtype."""
    w = np.zeros((D, ncols), dtype=np.float32)
    for c in range(ncols):
        rows = draw.rng.choice(D, size=min(nnz, D), replace=False)
        w[rows, c] = draw.rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=len(rows))
    return w


def draw_layer(seed: int, B: int, T: int, past, D: int, Hq: int, Hkv: int, d: int, dtype: str,
               cap: int, exact: bool = False, past_lo: int = 0, past_hi: int = 0):
    """All inputs of one layer step as float32 arrays exact in `dtype`:
    wq [D, Hq*d], wk/wv [D, Hkv*d], x [B, T, D], past_len int32 [B], and past caches
    kp/vp [B, Hkv, cap, d] holding rows [0, past_len[b]) (zeros elsewhere).
    exact=True draws integer X in [-8, 8] and sparse +-1 weights (exact projections)."""
    dr = Draw(seed)
    if exact:
        wq = sparse_sign_weights(dr, D, Hq * d)
        wk = sparse_sign_weights(dr, D, Hkv * d)
        wv = sparse_sign_weights(dr, D, Hkv * d)
    else:
        wq, wk, wv = layer_weights(dr, D, Hq, Hkv, d, dtype)
    past_len = dr.lengths(B, past_lo, past_hi) if past is None else np.asarray(past, dtype=np.int32)
    x = dr.integers((B, T, D), -8, 8) if exact else dr.normal((B, T, D), 1.0, dtype)
    kp = np.zeros((B, Hkv, cap, d), dtype=np.float32)
    vp = np.zeros((B, Hkv, cap, d), dtype=np.float32)
    fill_past(dr, kp, vp, past_len, dtype)
    return dict(wq=wq, wk=wk, wv=wv, x=x, past_len=past_len, kp=kp, vp=vp, dtype=dtype,
                B=B, T=T, D=D, Hq=Hq, Hkv=Hkv, d=d, cap=cap)


def grid(a: np.ndarray, step: float, lim: float) -> np.ndarray:
    """Values on the grid of multiples of `step`, clipped to [-lim, lim] (input encoding: with
    step and lim powers of two and lim/step <= 128, every value is exact in bf16, f16 and f32)."""
    return np.clip(np.round(np.asarray(a, dtype=np.float64) / step) * step, -lim, lim).astype(np.float32)


def draw_layer_large_scores(seed: int, B: int, T: int, past, D: int, Hq: int, Hkv: int, d: int, dtype: str,
                            cap: int, x_max: int = 16, k_lo: float = 0.5, k_hi: float = 4.0,
                            past_lo: int = 0, past_hi: int = 0):
    """Inputs with large attention scores that grow along the key positions, for the softmax's
    running maximum: it is raised again and again across key tiles and launches.

    Every stored input and every product the layer forms from them is exact in all three dtypes:
    X holds integers in [-x_max, x_max]; Wq has 8 entries of +-1 per column (so |Q| <= 8 x_max,
    integers); Wk and Wv have 8 entries of +-1/16 and +-1/32 per column; past K is N(0,1) times a
    ramp that grows geometrically from k_lo at key 0 to k_hi at the last past key, and past V is
    N(0,1), both on the grid of 1/16 within [-8, 8]. With x_max <= 16 the query-key dot products
    are multiples of 1/16 below 2^21, exact in fp32, so the only rounding in the scores is their
    scaling. Draw order: Wq, Wk, Wv, lengths (if ragged), X, past K, past V."""
    dr = Draw(seed)
    wq = sparse_sign_weights(dr, D, Hq * d)
    wk = sparse_sign_weights(dr, D, Hkv * d) / np.float32(16)
    wv = sparse_sign_weights(dr, D, Hkv * d) / np.float32(32)
    past_len = dr.lengths(B, past_lo, past_hi) if past is None else np.asarray(past, dtype=np.int32)
    x = dr.integers((B, T, D), -x_max, x_max)
    kp = np.zeros((B, Hkv, cap, d), dtype=np.float32)
    vp = np.zeros((B, Hkv, cap, d), dtype=np.float32)
    for b in range(B):
        L = int(past_len[b])
        ramp = (k_lo * (k_hi / k_lo) ** (np.arange(L) / max(L - 1, 1))).astype(np.float32)[:, None]
        for g in range(Hkv):
            kp[b, g, :L] = grid(dr.rng.standard_normal((L, d), dtype=np.float32) * ramp, 1 / 16, 8)
    for b in range(B):
        L = int(past_len[b])
        for g in range(Hkv):
            vp[b, g, :L] = grid(dr.rng.standard_normal((L, d), dtype=np.float32), 1 / 16, 8)
    return dict(wq=wq, wk=wk, wv=wv, x=x, past_len=past_len, kp=kp, vp=vp, dtype=dtype,
                B=B, T=T, D=D, Hq=Hq, Hkv=Hkv, d=d, cap=cap)
