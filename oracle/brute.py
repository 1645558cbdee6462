"""Brute-force cross-check of the oracle, for tiny layers only (pure Python).

TEST INFRASTRUCTURE ONLY. An independent second implementation of the same plain
definition as `oracle` (projection, append, causal grouped-query softmax attention),
written with different means so that a slip in one is unlikely to be repeated in the
other: projections in exact rational arithmetic (fractions.Fraction), the full masked
score matrix built explicitly, exp from the math module and every sum through
math.fsum (correctly rounded). Rounding to a storage dtype is done by searching the
representable neighbours exactly, not by scaling.
"""
from __future__ import annotations

import math
from fractions import Fraction

_FMT = {"f32": (24, -126, 127), "f16": (11, -14, 15), "bf16": (8, -126, 127)}


def representable_round(v: Fraction, dtype: str):
    """Nearest value of `dtype` to the exact rational v, ties to the even significand.
    Returns a Fraction, or +-inf as float when v rounds beyond the largest finite value."""
    p, emin, emax = _FMT[dtype]
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent of the leading bit: 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - (p - 1))        # spacing of the format around a
    lo = (a // q) * q                       # candidate below (or equal)
    hi = lo + q                             # candidate above
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:                                   # exact tie: pick the even significand
        r = lo if (lo / q) % 2 == 0 else hi
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > max_finite:
        return sign * math.inf
    return sign * r


def _frac(v) -> Fraction:
    return Fraction(float(v))


def rotate(vec, pos, theta):
    """Rotary embedding of one head vector (floats) at position pos: element i < d/2 and element
    i + d/2 turn together by pos * theta ** (-2 i / d) (math.cos / math.sin of a Python float)."""
    d = len(vec)
    half = d // 2
    out = list(vec)
    for i in range(half):
        a = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


def layer_step(x, wq, wk, wv, kc, vc, past_len, n_q_heads, dtype, rope_theta=0.0):
    """x nested [B][T][D]; w [D][cols]; kc/vc nested [B][Hkv][cap][d] of floats
    (modified in place). Returns out as nested [B][T][Hq][d] floats. With rope_theta, q and
    the new k are rotated (in floats) at positions past_len[b] + t before the rounding."""
    B, T, D = len(x), len(x[0]) if x else 0, len(x[0][0]) if x and x[0] else 0
    Hkv = len(kc[0])
    d = len(kc[0][0][0])
    G = n_q_heads // Hkv

    def proj(row, w, col):
        return sum((_frac(row[k]) * _frac(w[k][col]) for k in range(D)), Fraction(0))

    # projections (exact) and append (rounded exactly)
    for b in range(B):
        for t in range(T):
            for g in range(Hkv):
                kvec = [proj(x[b][t], wk, g * d + i) for i in range(d)]
                if rope_theta:
                    kvec = [Fraction(v) for v in rotate([float(v) for v in kvec], past_len[b] + t, rope_theta)]
                for i in range(d):
                    kval = representable_round(kvec[i], dtype)
                    vval = representable_round(proj(x[b][t], wv, g * d + i), dtype)
                    kc[b][g][past_len[b] + t][i] = float(kval)
                    vc[b][g][past_len[b] + t][i] = float(vval)

    out = [[[[0.0] * d for _ in range(n_q_heads)] for _ in range(T)] for _ in range(B)]
    for b in range(B):
        L = past_len[b]
        nk = L + T
        for h in range(n_q_heads):
            g = h // G
            q = [[float(proj(x[b][t], wq, h * d + i)) for i in range(d)] for t in range(T)]
            if rope_theta:
                q = [rotate(q[t], L + t, rope_theta) for t in range(T)]
            # full score matrix with the causal mask applied as -inf
            S = [[(math.fsum(q[t][i] * kc[b][g][j][i] for i in range(d)) / math.sqrt(d))
                  if j <= L + t else -math.inf for j in range(nk)] for t in range(T)]
            for t in range(T):
                m = max(S[t])
                w = [math.exp(s - m) if s != -math.inf else 0.0 for s in S[t]]
                l = math.fsum(w)
                for i in range(d):
                    out[b][t][h][i] = math.fsum(w[j] * vc[b][g][j][i] for j in range(nk)) / l
    return out


def decode_stack_step(h, layers, caches, past_len, n_q_heads, dtype, eps):
    """The decoder-stack decode step of `oracle.decode_stack_step`, for tiny shapes, with plain
    loops: h nested [B][D]; layers: dicts of nested [in][out] weight lists and [D] norm weights;
    caches: per layer (kc, vc) nested lists (modified in place). Every stored tensor is rounded
    exactly (representable_round of the correctly rounded float value), at the same points.
    Returns h as nested floats."""
    def rnd(v):
        return float(representable_round(_frac(v), dtype))

    def norm(row, g):
        ms = math.fsum(v * v for v in row) / len(row)
        s = math.sqrt(ms + eps)
        return [rnd(row[i] / s * g[i]) for i in range(len(row))]

    def matvec(row, w):      # row [K] times w [K][N], exact, then rounded once
        K, N = len(w), len(w[0])
        return [sum((_frac(row[k]) * _frac(w[k][n]) for k in range(K)), Fraction(0)) for n in range(N)]

    h = [[rnd(v) for v in row] for row in h]
    B = len(h)
    for lw, (kc, vc) in zip(layers, caches):
        a = [norm(h[b], lw["g_attn"]) for b in range(B)]
        o = layer_step([[a[b]] for b in range(B)], lw["wq"], lw["wk"], lw["wv"], kc, vc, past_len, n_q_heads, dtype)
        o = [[rnd(v) for head in o[b][0] for v in head] for b in range(B)]
        h = [[rnd(_frac(h[b][n]) + p) for n, p in enumerate(matvec(o[b], lw["wo"]))] for b in range(B)]
        m = [norm(h[b], lw["g_mlp"]) for b in range(B)]
        gu = [[rnd(v) for v in matvec(m[b], lw["w_gu"])] for b in range(B)]
        F = len(gu[0]) // 2
        act = [[rnd(gu[b][j] / (1.0 + math.exp(-gu[b][j])) * gu[b][F + j]) for j in range(F)] for b in range(B)]
        h = [[rnd(_frac(h[b][n]) + p) for n, p in enumerate(matvec(act[b], lw["w_down"]))] for b in range(B)]
    return h
