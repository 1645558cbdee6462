"""Large and growing attention scores against the oracle, through the C ABI.

The prefill softmax raises its reference maximum lazily (only when a tile's maximum exceeds it
by more than 2^8) and rescales the running output and sum when it does; the running state also
crosses launches. With N(0,1) inputs scores barely move past the first tile's maximum, so these
cases draw inputs (synth.draw_layer_large_scores) whose scores reach about +-550 in base-2 units
(about +-380 in natural units, against +-4 for N(0,1) inputs) and whose spread grows along the
key positions: the maximum of a query row is raised 8-11 times over a few thousand keys, in
several launches, and the scores of this step's new keys are large as well.

Every input and every query-key product is exact in the three dtypes, so the GPU's rounding of
Q to bf16/f16 for the matrix cores loses nothing and the parity tolerances apply unchanged:
max-abs 2e-2 and mean-abs 2e-3 for bf16/f16, 1e-5 for fp32, against the fp64 oracle. The new
K/V rows are exact too, so the appended rows are compared bit for bit."""
import numpy as np
import pytest

import synth
from gpu_case import GpuLayer, compare, oracle_step

pytestmark = pytest.mark.gpu


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype, k_lo=0.5, k_hi=4.0, past_lo=0, past_hi=0):
    hi = max(past) if past is not None else past_hi
    cap = ((hi + T + 63) // 64 + 1) * 64
    return synth.draw_layer_large_scores(seed, B, T, past, D, Hq, Hkv, d, dtype, cap, k_lo=k_lo, k_hi=k_hi,
                                         past_lo=past_lo, past_hi=past_hi)


PREFILL = [
    # B, T, past, D, Hq, Hkv, d, dtype, keys per super-chunk (None: the planner's)
    (1, 256, [6000], 256, 8, 2, 128, "bf16", None),
    (1, 256, [6000], 256, 8, 2, 128, "bf16", 1024),      # 6 past launches + the new keys
    (2, 200, [2500, 7000], 256, 4, 2, 128, "f16", 1024),
    (1, 100, [5000], 256, 16, 2, 64, "bf16", 2048),      # G = 8, d = 64
    (1, 130, [3000], 256, 8, 8, 64, "f32", 1024),        # G = 1, fp32
    (1, 97, [2100], 256, 8, 2, 128, "f32", 512),         # G = 4, fp32, d = 128
    (3, 64, [0, 700, 4100], 256, 8, 2, 128, "bf16", 1024),   # ragged, one empty past
    # one query tile per pair: the keys are split over workgroups and the states merged
    (1, 16, [7000], 256, 16, 2, 128, "bf16", None),
    (2, 32, [3000, 9000], 256, 8, 2, 128, "f16", None),
    (1, 40, [2500], 256, 4, 4, 64, "f32", None),
]


def _ids(s):
    return f"B{s[0]}-T{s[1]}-L{max(s[2])}-G{s[4] // s[5]}-d{s[6]}-{s[7]}-sk{s[8]}"


@pytest.mark.parametrize("two_launch", ["1", "0"], ids=["two-launch", "per-chunk"])
@pytest.mark.parametrize("shape", PREFILL, ids=_ids)
def test_prefill_large_growing_scores(shape, two_launch, monkeypatch):
    """Both multi-super-chunk paths: the two-launch prefill (each super-chunk's state kept apart,
    merged at the end) and the launch-per-super-chunk path (one running state carried along)."""
    B, T, past, D, Hq, Hkv, d, dtype, sk = shape
    monkeypatch.setenv("DIRECTKV_PREFILL_CHUNKED", two_launch)
    if sk is not None:
        monkeypatch.setenv("DIRECTKV_PREFILL_CHUNK", str(sk))
    case = _case(31, B, T, past, D, Hq, Hkv, d, dtype)
    print(f"prefill {_ids(shape)}", flush=True)
    g = GpuLayer(case)
    try:
        out = g.prefill(case["x"], case["past_len"])
        kg, vg = g.cache.k.copy(), g.cache.v.copy()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(out, ref, dtype, f"prefill {_ids(shape)}")
    for b in range(B):
        L = int(case["past_len"][b])
        assert np.array_equal(kg[b, :, L:L + T], synth.to_storage(kc[b, :, L:L + T], dtype)), "K rows"
        assert np.array_equal(vg[b, :, L:L + T], synth.to_storage(vc[b, :, L:L + T], dtype)), "V rows"


def test_prefill_large_shrinking_scores(monkeypatch):
    """The spread shrinks along the keys: the maximum is set in the first tiles and the later
    tiles never raise it (the path where whole waves skip the rescale)."""
    monkeypatch.setenv("DIRECTKV_PREFILL_CHUNK", "1024")
    case = _case(32, 1, 160, [4000], 256, 8, 2, 128, "bf16", k_lo=4.0, k_hi=0.25)
    g = GpuLayer(case)
    try:
        out = g.prefill(case["x"], case["past_len"])
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    compare(out, oracle_step(case, case["x"], case["past_len"], kc, vc), "bf16", "prefill, shrinking scores")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_large_growing_scores(dtype):
    """Ragged decode over several splits per sequence with large, growing scores; the new
    token's own key and the appended row (bitwise) as well."""
    case = _case(33, 3, 1, [3000, 9000, 20000], 256, 8, 2, 128, dtype)
    g = GpuLayer(case)
    try:
        out = g.decode(case["x"], case["past_len"])
        kg = g.cache.k.copy()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(out, ref, dtype, f"decode {dtype}")
    for b in range(3):
        L = int(case["past_len"][b])
        assert np.array_equal(kg[b, :, L], synth.to_storage(kc[b, :, L], dtype))
