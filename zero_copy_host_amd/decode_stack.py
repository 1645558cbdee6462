"""A stack of decoder layers for the decode step, each layer with its own host KV cache.

Per layer (pre-norm block): h <- h + attn(rmsnorm(h)) Woᵀ, h <- h + swiglu(rmsnorm(h) W_guᵀ) W_downᵀ,
where attn is the library's host-KV attention layer step (q/k/v projection, rotary embedding of q
and k when rope_theta > 0, append of the new token's K/V to the host cache, causal GQA attention
over it) and the rest are the library's decode-loop kernels. This module only sequences the C-ABI calls and owns the scratch buffers;
every step runs in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from . import HostKVCache, attn_decode, linear, rmsnorm, swiglu, workspace_bytes


class DecodeStack:
    """`layers`: per layer, device tensors in [out, in] layout — wq [Hq·d, D], wk and wv
    [Hkv·d, D], wo [D, Hq·d], w_gu [2F, D] (gate rows, then up rows), w_down [D, F] — and the
    norm weights g_attn, g_mlp [D]. `caches`: one HostKVCache per layer (same batch, heads,
    head_dim and dtype)."""

    def __init__(self, layers: List[Dict], caches: Sequence[HostKVCache], n_q_heads: int, eps: float = 1e-5,
                 rope_theta: float = 0.0):
        import torch
        if len(layers) != len(caches) or not layers:
            raise ValueError("one cache per layer, at least one layer")
        self.layers, self.caches, self.Hq, self.eps = layers, list(caches), n_q_heads, eps
        self.rope_theta = rope_theta   # rotary base for q and k (0: none, the layer as the pages give it)
        c = self.caches[0]
        self.B, self.d = c.batch, c.head_dim
        w0 = layers[0]
        self.D = w0["wq"].shape[1]
        self.F = w0["w_down"].shape[1]
        self.dtype = w0["wq"].dtype
        dev = w0["wq"].device
        B = self.B
        self.a = torch.empty((B, 1, self.D), dtype=self.dtype, device=dev)          # normed input
        self.o = torch.empty((B, 1, n_q_heads * self.d), dtype=self.dtype, device=dev)  # attention out
        self.gu = torch.empty((B, 2 * self.F), dtype=self.dtype, device=dev)
        self.act = torch.empty((B, self.F), dtype=self.dtype, device=dev)
        self.ws = torch.empty(workspace_bytes("decode", c, B, 1, n_q_heads), dtype=torch.uint8, device=dev)

    def step(self, h, past_len) -> None:
        """One decode step for every sequence; h [B, D] is updated in place. The new token's K/V of
        every layer are appended at row past_len[b] of that layer's cache."""
        past = np.asarray(past_len, dtype=np.int32)
        for lw, cache in zip(self.layers, self.caches):
            rmsnorm(h, lw["g_attn"], self.a, self.eps)
            attn_decode(cache, self.a, lw["wq"], lw["wk"], lw["wv"], past, self.Hq, self.o, self.ws,
                        rope_theta=self.rope_theta)
            linear(self.o, lw["wo"], h, residual=h)
            rmsnorm(h, lw["g_mlp"], self.a, self.eps)
            linear(self.a, lw["w_gu"], self.gu)
            swiglu(self.gu, self.act)
            linear(self.act, lw["w_down"], h, residual=h)
