"""Host-side accounting: pinned to the pages' printed worked example and to closed forms."""
import json
import os

import pytest

from zero_copy_host_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes_page4.json")


def test_kv_bytes_per_token_matches_page_example():
    g = json.load(open(GOLDEN))
    m = g["model"]
    b = acc.kv_bytes_per_token(m["layers"], m["n_kv_heads"], m["head_dim"], m["elem_bytes"])
    assert b == g["bytes_per_token_printed_KiB"] * 1024


def test_fetch_times_match_page_example():
    g = json.load(open(GOLDEN))
    m = g["model"]
    b = acc.kv_bytes_per_token(m["layers"], m["n_kv_heads"], m["head_dim"], m["elem_bytes"])
    for c in g["cases"]:
        ms = acc.fetch_seconds(c["tokens"], b, c["GBps"] * 1e9) * 1e3
        assert abs(ms - c["printed_ms"]) <= 0.03 * c["printed_ms"], c
    assert abs(1000 * b / 1e6 - 160) <= 0.03 * 160
    assert abs(20000 * b / 1e9 - 3.2) <= 0.03 * 3.2


def test_layer_step_bytes_and_flops():
    # 8B-shaped decode: B=8, 32768 past tokens, Hkv=8, d=128, bf16 -> exactly 1 GiB read
    assert acc.host_read_bytes([32768] * 8, 8, 128, 2) == 1 << 30
    assert acc.host_write_bytes(8, 1, 8, 128, 2) == 32768
    # one token attending to L+1 keys: 4*d*Hq*(L+1)
    assert acc.attention_flops([10], 1, 4, 64) == 4 * 64 * 4 * 11
    # causal block of T new tokens on an empty cache: T(T+1)/2 pairs
    assert acc.attention_flops([0], 5, 1, 2) == 4 * 2 * 15
    assert acc.projection_flops(1, 3, 16, 4, 2, 8) == 2 * 3 * 16 * (4 + 4) * 8


def test_smem_rule():
    # closed form of alpha*P >= 3*m*e*Dim*N: 0.8 * 256 KiB / (3*2*2*128) = 136.53
    assert acc.smem_max_tile(256 * 1024, 0.8, 2, 2, 128) == 136
    assert acc.smem_max_tile(160 * 1024, 1.0, 2, 2, 128) == 106
    assert acc.smem_max_tile(160 * 1024, 1.0, 3, 2, 128) == 71


def _simulate_two_stage(n, comp, xfer):
    """Event simulation: one producer, one consumer, two buffers."""
    t_xfer_done = []
    free = [0.0, 0.0]           # time each buffer becomes free
    prod_t = 0.0
    cons_t = 0.0
    for i in range(n):
        start = max(prod_t, free[i % 2])
        prod_t = start + xfer
        t_xfer_done.append(prod_t)
        cstart = max(cons_t, prod_t)
        cons_t = cstart + comp
        free[i % 2] = cons_t
    return cons_t


@pytest.mark.parametrize("n,comp,xfer", [(1, 120, 100), (7, 120, 100), (9, 80, 100), (5, 50, 50)])
def test_pipeline_model_matches_event_simulation(n, comp, xfer):
    assert acc.pipeline_cycles(n, comp, xfer) == pytest.approx(_simulate_two_stage(n, comp, xfer))


def test_overlap_model_limits():
    # link-bound stream: the whole transfer plus one tile's compute
    assert acc.overlap_model_seconds(100, 1e9, 1e6, 1e10, 1e12) == pytest.approx(0.1 + 1e-6 / 100)
    # compute-bound stream: one tile's transfer plus the whole compute
    assert acc.overlap_model_seconds(50, 1e6, 1e12, 1e10, 1e12) == pytest.approx(1e-4 / 50 + 1.0)
    # one tile: no overlap at all
    assert acc.overlap_model_seconds(1, 1e9, 1e12, 1e10, 1e12) == pytest.approx(0.1 + 1.0)
    assert acc.overlap_model_seconds(0, 1e9, 1e12, 1e10, 1e12) == 0.0
