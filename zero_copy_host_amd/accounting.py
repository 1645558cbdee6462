"""Algorithmic bytes and flops of one layer step, and the pages' sizing rules.

Used by the benchmark for rooflines. No kernel arithmetic lives here.
"""
from __future__ import annotations

from typing import Sequence


def kv_bytes_per_token(layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one token occupies across `layers` layers: 2 * layers * h_kv * d * bytes
    ("KV Offloading and Transfer", section 2, the fetch-cost formula)."""
    return 2 * layers * n_kv_heads * head_dim * elem_bytes


def fetch_seconds(tokens: int, bytes_per_token: int, bandwidth_bytes_per_s: float) -> float:
    """Time to move the KV of `tokens` tokens over a link (same section)."""
    return tokens * bytes_per_token / bandwidth_bytes_per_s


def host_read_bytes(past_len: Sequence[int], n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Past K and V rows one layer step reads from the host cache, each exactly once."""
    return kv_bytes_per_token(1, n_kv_heads, head_dim, elem_bytes) * int(sum(int(x) for x in past_len))


def host_write_bytes(batch: int, new_tokens: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """New K and V rows one layer step appends to the host cache."""
    return kv_bytes_per_token(1, n_kv_heads, head_dim, elem_bytes) * batch * new_tokens


def attention_flops(past_len: Sequence[int], new_tokens: int, n_q_heads: int, head_dim: int) -> int:
    """QKᵀ and PV multiply-adds (2 flops each) of causal attention: token t of sequence b sees
    past_len[b] + t + 1 keys."""
    T = new_tokens
    pairs = sum(T * int(L) + T * (T + 1) // 2 for L in past_len)
    return 4 * head_dim * n_q_heads * pairs


def projection_flops(batch: int, new_tokens: int, D: int, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    """X·Wqᵀ, X·Wkᵀ and X·Wvᵀ for the new tokens."""
    return 2 * batch * new_tokens * D * (n_q_heads + 2 * n_kv_heads) * head_dim


def smem_max_tile(pool_bytes: int, alpha: float, stages: int, elem_bytes: int, dim: int) -> int:
    """Largest tile N with alpha * P >= 3 * m * size(T) * Dim * N ("Paper Notes: DirectKV",
    System Architecture: three operand tiles per pipeline stage must fit the on-chip pool)."""
    return int((alpha * pool_bytes) // (3 * stages * elem_bytes * dim))


def pipeline_cycles(n_tiles: int, compute: float, transfer: float) -> float:
    """Two-stage producer/consumer time: the first transfer, then n-1 overlapped steps
    bounded by the slower of the two, then the last compute ("DirectKV Guide", warp-level
    pipelining)."""
    if n_tiles <= 0:
        return 0.0
    return transfer + (n_tiles - 1) * max(compute, transfer) + compute


def overlap_model_seconds(n_tiles: int, host_bytes: float, flops: float, link_bytes_per_s: float,
                          compute_flops_per_s: float) -> float:
    """Expected time of one step under the two-stage pipeline model of the "DirectKV Guide"
    (warp-level pipelining): the step's host bytes and flops are spread evenly over the
    `n_tiles` key tiles of one stream, a tile's transfer runs at the link rate and its compute
    at the compute rate, and the stream pays the first transfer, n - 1 overlapped tiles and the
    last compute."""
    if n_tiles <= 0:
        return 0.0
    transfer = host_bytes / n_tiles / link_bytes_per_s
    compute = flops / n_tiles / compute_flops_per_s
    return pipeline_cycles(n_tiles, compute, transfer)
