"""The two-launch prefill (a chunk launch of every past super-chunk's items, each leaving its own
running state, then a finish launch whose own-key items fold every state in) against the oracle
and against the launch-per-super-chunk path, through the C ABI.

Super-chunks are forced small (DIRECTKV_PREFILL_CHUNK) so that a few hundred past keys make many
of them, with ragged and empty past lengths, all three dtypes and both head sizes. The dispatch
order (DIRECTKV_PREFILL_INSERT) changes no bit; where the own-key items run
(DIRECTKV_PREFILL_OWN) changes the merge order only, so those runs are held to the oracle."""
import numpy as np
import pytest

import synth
from gpu_case import GpuLayer, absdot_rows, compare, compare_rows, oracle_step

pytestmark = pytest.mark.gpu


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype):
    cap = ((max(past) + T + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap)


def _run(case, env, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    g = GpuLayer(case, canary=True)
    try:
        out = g.prefill(case["x"], case["past_len"])
        kg, vg = g.cache_k(), g.cache_v()
    finally:
        g.free()
    return out, kg, vg


CASES = [
    # B, T, past, D, Hq, Hkv, d, dtype, keys per super-chunk
    (2, 300, [1000, 0], 512, 8, 2, 128, "bf16", 256),        # 4 pairs, 5 query tiles, 4 super-chunks
    (3, 100, [700, 1500, 33], 256, 16, 2, 64, "f16", 256),   # G = 8, d = 64, ragged, 6 super-chunks
    (1, 260, [900], 256, 4, 4, 64, "f32", 192),              # G = 1, fp32, 5 super-chunks
    (1, 200, [2000], 256, 32, 8, 128, "bf16", 256),          # 8 pairs, one per XCD, 8 super-chunks
    (2, 150, [1300, 640], 256, 32, 8, 128, "f16", 320),      # 16 pairs: two groups of 8
    (1, 97, [2100], 256, 8, 2, 128, "f32", 512),             # G = 4, fp32, d = 128
    (3, 130, [2600, 1200, 0], 256, 16, 4, 64, "bf16", 256),  # 12 pairs, 2 per XCD's L2, 11 super-chunks
    (2, 520, [900, 1800], 256, 8, 1, 128, "bf16", 128),      # G = 8, 17 query tiles, 15 super-chunks
    (1, 64, [2000], 256, 8, 2, 128, "bf16", 256),            # T*G = 256: one query tile, key splits instead
    (1, 65, [2000], 256, 8, 2, 128, "bf16", 256),            # T*G = 260: two query tiles, the last of 4 rows
]


def _ids(s):
    return f"B{s[0]}-T{s[1]}-L{max(s[2])}-G{s[4] // s[5]}-d{s[6]}-{s[7]}-sk{s[8]}"


@pytest.mark.parametrize("shape", CASES, ids=_ids)
def test_two_launch_prefill_parity(shape, monkeypatch):
    B, T, past, D, Hq, Hkv, d, dtype, sk = shape
    print(f"two-launch prefill {_ids(shape)}", flush=True)
    case = _case(41, B, T, past, D, Hq, Hkv, d, dtype)
    out, kg, vg = _run(case, {"DIRECTKV_PREFILL_CHUNK": str(sk), "DIRECTKV_PREFILL_CHUNKED": "1"}, monkeypatch)
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(out, ref, dtype, f"two-launch {_ids(shape)}")
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in range(B):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L:L + T], kc[b, :, L:L + T], dtype, ak[b], D, "new K rows")
        compare_rows(vg[b, :, L:L + T], vc[b, :, L:L + T], dtype, av[b], D, "new V rows")
        # nothing past the new rows is written
        assert np.isnan(kg[b, :, L + T:]).all() and np.isnan(vg[b, :, L + T:]).all()
    # the launch-per-super-chunk path on the same inputs: also within tolerance of the oracle, and
    # the same appended rows bit for bit
    out0, kg0, vg0 = _run(case, {"DIRECTKV_PREFILL_CHUNK": str(sk), "DIRECTKV_PREFILL_CHUNKED": "0"}, monkeypatch)
    compare(out0, ref, dtype, f"per-chunk {_ids(shape)}")
    for b in range(B):
        L = int(case["past_len"][b])
        assert np.array_equal(kg[b, :, L:L + T], kg0[b, :, L:L + T])
        assert np.array_equal(vg[b, :, L:L + T], vg0[b, :, L:L + T])


def test_dispatch_order_changes_no_bit(monkeypatch):
    """The insertion point of the next super-chunk's fetchers only reorders independent items."""
    shape = CASES[3]
    B, T, past, D, Hq, Hkv, d, dtype, sk = shape
    case = _case(42, B, T, past, D, Hq, Hkv, d, dtype)
    outs = []
    for ins in ("0", "3", "1000"):
        out, _, _ = _run(case, {"DIRECTKV_PREFILL_CHUNK": str(sk), "DIRECTKV_PREFILL_INSERT": ins}, monkeypatch)
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("own", ["0", "50", "100"])
def test_own_key_split_between_launches(own, monkeypatch):
    """Own-key items all in the finish launch (0), half the work in the chunk launch, or all of
    them there (100, the finish launch then only merges)."""
    shape = CASES[1]
    B, T, past, D, Hq, Hkv, d, dtype, sk = shape
    case = _case(43, B, T, past, D, Hq, Hkv, d, dtype)
    out, _, _ = _run(case, {"DIRECTKV_PREFILL_CHUNK": str(sk), "DIRECTKV_PREFILL_OWN": own}, monkeypatch)
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(out, ref, dtype, f"own={own}%")
