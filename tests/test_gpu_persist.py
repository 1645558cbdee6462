"""The persistent prefill (DKV_PREFILL_PERSIST: one launch per group of 8 pairs, a work queue
per XCD, a producer that streams the next key super-chunk while the current one is computed,
the running state handed between items of a query tile through completion counters) against
the oracle, through the C ABI, with the tolerances of the fused path. Its super-chunks are half
the fused path's size, so the results are not bit-identical to attn_prefill; they are
deterministic (a fixed order per query tile) and the appended rows are the same."""
import numpy as np
import pytest

import synth
from gpu_case import GpuLayer, absdot_rows, compare, compare_rows, oracle_step

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="DKV_PREFILL_PERSIST is disabled: its launch did not complete on the GPU (the "
                            "first case ran past its time limit twice, the second time with every wait "
                            "bounded); the ABI refuses the variant until the cause is found"),
]


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype):
    cap = ((max(past) + T + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap)


CASES = [
    # B, T, past, D, Hq, Hkv, d, dtype
    (1, 300, [3000], 256, 32, 8, 128, "bf16"),          # 8 pairs, 5 query tiles, 2 super-chunks
    (2, 300, [3000, 4500], 256, 32, 8, 128, "bf16"),    # 16 pairs: two persistent launches
    (1, 1100, [5000], 256, 32, 8, 128, "f16"),          # 18 query tiles, 4 super-chunks
    (1, 2048, [2100], 256, 16, 8, 64, "bf16"),          # G = 2, d = 64: 16 query tiles
    (4, 64, [0, 1000, 64, 2200], 256, 8, 2, 128, "bf16"),  # ragged lengths across the group
    (1, 130, [700], 256, 8, 8, 64, "f32"),               # G = 1, fp32
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: f"B{s[0]}-T{s[1]}-L{max(s[2])}-G{s[4]//s[5]}-d{s[6]}-{s[7]}")
def test_persistent_prefill_parity(shape):
    B, T, past, D, Hq, Hkv, d, dtype = shape
    case = _case(21, B, T, past, D, Hq, Hkv, d, dtype)
    g = GpuLayer(case, canary=True)
    try:
        out = g.prefill(case["x"], case["past_len"], variant="persistent")
        kg, vg = g.cache_k(), g.cache_v()
        again = g.prefill(case["x"], case["past_len"], variant="persistent")   # same rows rewritten
    finally:
        g.free()
    assert np.array_equal(out.view(np.uint8), again.view(np.uint8)), "reruns differ"
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(out, ref, dtype, f"persistent prefill {shape}")
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in range(B):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L:L + T], kc[b, :, L:L + T], dtype, ak[b], D, "new K rows")
        compare_rows(vg[b, :, L:L + T], vc[b, :, L:L + T], dtype, av[b], D, "new V rows")


def test_persistent_prefill_appends_the_same_rows_as_the_fused_path():
    case = _case(22, 2, 200, [1000, 2500], 256, 32, 8, 128, "bf16")
    rows = {}
    for variant in (None, "persistent"):
        g = GpuLayer(case)
        try:
            g.prefill(case["x"], case["past_len"], variant=variant)
            rows[variant] = (g.cache.k.copy(), g.cache.v.copy())
        finally:
            g.free()
    for b, L in enumerate(case["past_len"]):
        for i in range(2):
            assert np.array_equal(rows[None][i][b, :, :L + 200], rows["persistent"][i][b, :, :L + 200])
