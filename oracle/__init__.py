"""Oracle: a plain, slow fp64 CPU implementation of one host-KV attention layer step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
package; only the tests, the package's smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library. The same layer step (without the
rotary embedding) is also written as plain threaded C loops in layer_ref.c (bound by
oracle.cref): the form the CPU baseline times, pinned against this one and the brute force.

What it computes (the plain definition; the method reaches the same result, only with a
different memory layout and transfer schedule — "DirectKV Guide: Zero-Copy KV
Offloading on GH200 & GB200", FAQ, on the method being lossless):

1. Projections without bias, K = X·Wk and V = X·Wv (and Q = X·Wq, the query the
   attention uses) — "Paper Notes: DirectKV", section "Fundamental Underlying
   Technologies / Kernel Fusion (Projection + Attention)", step 1 of the standard path.
2. The new K/V rows go into the KV cache held in host memory, where they stay and are
   reused by later steps — same page, section "System Architecture", KV Cache Manager.
3. Attention softmax(Q·Kᵀ/√d)·V over every cached key a query may see — same page,
   "Kernel Fusion", step 2 of the standard path.

Where the pages leave a step open, the readings taken are:
- scale 1/√d (given on "Paper Notes: DirectKV"; the guide's formula drops it);
- grouped-query attention: query head h reads KV head h // G, G = Hq / Hkv;
- causal alignment: new token t of sequence b sits at absolute position past_len[b] + t
  and sees keys 0 .. past_len[b] + t, itself included (a decode step attends to the key
  it has just appended);
- no bias and no output projection, and no RoPE in the layer as the pages give it
  (rope_theta = 0; the rotary embedding below serves the decoder stack around the layer);
  W is stored [D, H·d] and applied as X·W; head h occupies columns [h·d, (h+1)·d);
- rounding happens only where the layer stores: appended cache rows are rounded to the
  cache dtype (round to nearest, ties to even) and the attention reads the rounded
  rows; Q and the output are kept in fp64 here.

Arrays: X [B, T, D]; Wq [D, Hq·d]; Wk, Wv [D, Hkv·d]; caches [B, Hkv, cap, d]
(float32 arrays whose values are exact in the cache dtype, or fp64); past_len int [B].

Rotary position embedding (for the decoder stack around the layer; the pages' layer has none):
with rope_theta > 0, q and the new k are rotated at their absolute positions before the attention
and the append. Pairs (i, i + d/2) of each head, i < d/2, turn by the angle p * theta^(-2i/d):
  y_i = x_i cos - x_{i+d/2} sin,  y_{i+d/2} = x_{i+d/2} cos + x_i sin,
the rotate-half form of the common Llama-family decoder.

A paged cache (16-token pages and a table from a sequence's logical pages to physical
pages — "DirectKV Guide: Zero-Copy KV Offloading on GH200 & GB200", section "End-to-End
Implementation: Building DirectKV in Python", its memory configuration and page manager)
holds the same logical cache: gather_pages gives it back, and the layer step on a paged
cache is the layer step above on the gathered cache.
"""
from __future__ import annotations

import numpy as np

# significand precision p (hidden bit included), minimum normal exponent, maximum exponent
_FORMATS = {"f32": (24, -126, 127), "f16": (11, -14, 15), "bf16": (8, -126, 127)}


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest value representable in `dtype`, ties to even
    (IEEE 754 roundTiesToEven), with gradual underflow and overflow to infinity.
    Returns fp64 holding the rounded values."""
    p, emin, emax = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    sel = np.isfinite(x) & (x != 0.0)
    xs = x[sel]
    _, e2 = np.frexp(xs)                      # xs = m·2^e2, 1/2 <= |m| < 1
    lead = np.maximum(e2 - 1, emin)           # exponent of the leading bit; subnormals clamp
    quantum = np.ldexp(1.0, lead - (p - 1))   # spacing of representable values there
    r = np.rint(xs / quantum) * quantum       # exact scaling; rint rounds ties to even
    max_finite = np.ldexp(2.0 - 2.0 ** (1 - p), emax)
    r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, xs), r)
    out[sel] = r
    return out


def project(x, w) -> np.ndarray:
    """X·W in fp64 (library matrix product). x [..., D], w [D, n] -> [..., n]."""
    return np.matmul(np.asarray(x, dtype=np.float64), np.asarray(w, dtype=np.float64))


def append(cache: np.ndarray, rows, past_len, dtype: str) -> None:
    """Write rows [B, T, H, d] into cache [B, H, cap, d] at token rows
    [past_len[b], past_len[b] + T), rounded to `dtype`. Nothing else is touched."""
    rows = np.asarray(rows, dtype=np.float64)
    B, T, H, d = rows.shape
    cap = cache.shape[2]
    assert cache.shape == (B, H, cap, d)
    for b in range(B):
        p = int(past_len[b])
        if p < 0 or p + T > cap:
            raise ValueError(f"append beyond capacity: past_len={p} T={T} cap={cap}")
        for g in range(H):
            cache[b, g, p:p + T, :] = round_to_dtype(rows[b, :, g, :], dtype)


def attention(q, kc, vc, past_len, t_index=None, return_lse: bool = False):
    """Causal grouped-query attention over the cache.

    q [B, n, Hq, d] holds the queries of new tokens t_index[0..n) (default 0..n-1);
    token t of sequence b sees cache rows 0 .. past_len[b] + t. Returns O [B, n, Hq, d]
    in fp64 (and log-sum-exp of the scaled scores, [B, n, Hq], if asked)."""
    q = np.asarray(q, dtype=np.float64)
    B, n, Hq, d = q.shape
    Hkv = kc.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    ts = np.arange(n) if t_index is None else np.asarray(t_index, dtype=np.int64)
    out = np.zeros((B, n, Hq, d), dtype=np.float64)
    lse = np.zeros((B, n, Hq), dtype=np.float64)
    if n == 0:
        return (out, lse) if return_lse else out
    for b in range(B):
        L = int(past_len[b])
        nkeys = L + int(ts.max()) + 1
        for g in range(Hkv):
            K = np.asarray(kc[b, g, :nkeys, :], dtype=np.float64)
            V = np.asarray(vc[b, g, :nkeys, :], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                for r, t in enumerate(ts):
                    p = L + int(t)                         # absolute position of the query
                    s = (K[: p + 1] @ q[b, r, h]) / np.sqrt(d)
                    m = s.max()
                    w = np.exp(s - m)
                    l = w.sum()
                    out[b, r, h] = (w @ V[: p + 1]) / l
                    lse[b, r, h] = m + np.log(l)
    return (out, lse) if return_lse else out


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotary position embedding of x [B, n, H, d] at absolute positions [B, n], in fp64:
    pair (i, i + d/2) of every head turns by positions * theta^(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)          # [d/2]
    ang = np.asarray(positions, dtype=np.float64)[..., None, None] * inv_freq          # [B, n, 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def layer_step(x, wq, wk, wv, kc, vc, past_len, n_q_heads: int, dtype: str, t_index=None,
               rope_theta: float = 0.0):
    """One layer step: project K/V of the T new tokens, append them to the caches
    (modified in place), then attend for the new tokens t_index (default all).
    With rope_theta > 0, q and the new k are rotated at positions past_len[b] + t first.
    Returns O [B, n, Hq, d] in fp64."""
    x = np.asarray(x)
    B, T, D = x.shape
    Hkv, d = kc.shape[1], kc.shape[3]
    kn = project(x, wk).reshape(B, T, Hkv, d)
    vn = project(x, wv).reshape(B, T, Hkv, d)
    pos = np.asarray(past_len, dtype=np.int64)[:, None] + np.arange(T)[None, :]          # [B, T]
    if rope_theta:
        kn = rope(kn, pos, rope_theta)
    append(kc, kn, past_len, dtype)
    append(vc, vn, past_len, dtype)
    ts = np.arange(T) if t_index is None else np.asarray(t_index, dtype=np.int64)
    q = project(x[:, ts, :], wq).reshape(B, len(ts), n_q_heads, d)
    if rope_theta:
        q = rope(q, pos[:, ts], rope_theta)
    return attention(q, kc, vc, past_len, ts)


PAGE_TOKENS = 16   # tokens per page of a paged cache (the page manager's page size)


def gather_pages(pool, table, n_tokens) -> np.ndarray:
    """The logical cache held by a paged pool.

    pool [n_pages, H, 16, d]; table int [B, max_pages] (logical page p of sequence b is
    physical page table[b, p]); n_tokens int [B]. Returns fp64 [B, H, max(n_tokens), d]:
    row j < n_tokens[b] of (sequence b, head g) is pool[table[b, j // 16], g, j % 16];
    rows at or past n_tokens[b] are NaN."""
    pool = np.asarray(pool, dtype=np.float64)
    table = np.asarray(table)
    B = table.shape[0]
    H, d = pool.shape[1], pool.shape[3]
    n = int(max(n_tokens)) if B else 0
    out = np.full((B, H, n, d), np.nan)
    for b in range(B):
        j = np.arange(int(n_tokens[b]))
        rows = pool[table[b, j // PAGE_TOKENS], :, j % PAGE_TOKENS, :]   # [len(j), H, d]
        out[b, :, : len(j), :] = rows.transpose(1, 0, 2)
    return out


# ---- a stack of decoder layers around the layer step (the decode loop's surroundings; the
# pages describe the attention layer only, so these follow the common pre-norm decoder block)

def rmsnorm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)


def silu(z) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + e^-z), in fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gu) -> np.ndarray:
    """silu(gate) * up for gu = [gate, up] side by side on the last axis."""
    gu = np.asarray(gu, dtype=np.float64)
    F = gu.shape[-1] // 2
    return silu(gu[..., :F]) * gu[..., F:]


def decode_stack_step(h, layers, caches, past_len, n_q_heads: int, dtype: str, eps: float,
                      rope_theta: float = 0.0) -> np.ndarray:
    """One decode step of a stack of pre-norm decoder layers on hidden states h [B, D]:
    h <- h + attn(rmsnorm(h)) @ Wo;  h <- h + swiglu(rmsnorm(h) @ W_gu) @ W_down.
    layers: dicts of [in, out] weights (wq, wk, wv, wo, w_gu, w_down, g_attn, g_mlp);
    caches: one (kc, vc) pair per layer, appended to in place. Every tensor the GPU stores
    between kernels (each norm output, the attention output, each residual sum, the MLP's
    gate-up product and activation) is rounded to `dtype` here at the same points."""
    h = round_to_dtype(h, dtype)
    B, D = h.shape
    for lw, (kc, vc) in zip(layers, caches):
        a = round_to_dtype(rmsnorm(h, lw["g_attn"], eps), dtype)
        o = layer_step(a[:, None, :], lw["wq"], lw["wk"], lw["wv"], kc, vc, past_len, n_q_heads, dtype,
                       rope_theta=rope_theta)
        o = round_to_dtype(o.reshape(B, -1), dtype)
        h = round_to_dtype(h + project(o, lw["wo"]), dtype)
        m = round_to_dtype(rmsnorm(h, lw["g_mlp"], eps), dtype)
        gu = round_to_dtype(project(m, lw["w_gu"]), dtype)
        act = round_to_dtype(swiglu(gu), dtype)
        h = round_to_dtype(h + project(act, lw["w_down"]), dtype)
    return h

