"""Parity of the HIP path (through the C ABI) with the oracle, on seeded synthetic inputs.

Small cases span several tiles, several decode splits, several prefill super-chunks and
ragged tails; exact-arithmetic cases check the append bit for bit; invariants check
properties the oracle also satisfies (causal perturbation, determinism, phase
consistency).
"""
import numpy as np
import pytest

import synth
from gpu_case import GpuLayer, absdot_rows, compare, compare_rows, oracle_step

pytestmark = pytest.mark.gpu


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype, cap=None, exact=False, past_lo=0, past_hi=0):
    if cap is None:
        hi = max(past) if past is not None else past_hi
        cap = ((hi + T + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap, exact=exact,
                            past_lo=past_lo, past_hi=past_hi)


def _run_prefill(case, t_index=None, canary=False):
    g = GpuLayer(case, canary=canary)
    try:
        out = g.prefill(case["x"], case["past_len"])
        kc_g, vc_g = g.cache_k(), g.cache_v()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc, t_index=t_index)
    if t_index is not None:
        out = out[:, t_index]
    return out, ref, kc_g, vc_g, kc, vc


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_exact_bitwise_with_canaries(dtype, d):
    """Exact-arithmetic inputs: appended rows equal the oracle bit for bit; every other
    row (past rows and NaN canaries) is untouched."""
    case = _case(11, 3, 37, [5, 0, 130], 256, 4, 2, d, dtype, exact=True)
    g = GpuLayer(case, canary=True)
    try:
        before_k, before_v = g.cache.k.copy(), g.cache.v.copy()
        g.append(case["x"], case["past_len"])
        kg, vg = g.cache.k.copy(), g.cache.v.copy()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    import oracle
    B, T = case["B"], case["T"]
    kn = oracle.project(case["x"], case["wk"]).reshape(B, T, case["Hkv"], d)
    vn = oracle.project(case["x"], case["wv"]).reshape(B, T, case["Hkv"], d)
    oracle.append(kc, kn, case["past_len"], dtype)
    oracle.append(vc, vn, case["past_len"], dtype)
    for b in range(B):
        L = int(case["past_len"][b])
        rows = slice(L, L + T)
        assert np.array_equal(kg[b, :, rows], synth.to_storage(kc[b, :, rows], dtype))
        assert np.array_equal(vg[b, :, rows], synth.to_storage(vc[b, :, rows], dtype))
        for arr_g, arr_b in ((kg, before_k), (vg, before_v)):
            assert np.array_equal(arr_g[b, :, :L].view(np.uint8), arr_b[b, :, :L].view(np.uint8))
            assert np.array_equal(arr_g[b, :, L + T:].view(np.uint8), arr_b[b, :, L + T:].view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [192, 320])
def test_append_exact_odd_reduction_steps(dtype, D):
    """D = 192 and 320 give the projection 3 and 5 reduction steps of 64: the loop's odd
    last step, and operand loads issued past the last step, against exact-arithmetic inputs
    (bitwise), with the rows around the appended ones untouched."""
    case = _case(15, 2, 45, [3, 100], D, 4, 2, 64, dtype, exact=True)
    g = GpuLayer(case, canary=True)
    try:
        before_k = g.cache.k.copy()
        g.append(case["x"], case["past_len"])
        kg, vg = g.cache.k.copy(), g.cache.v.copy()
    finally:
        g.free()
    import oracle
    B, T, Hkv, d = case["B"], case["T"], case["Hkv"], case["d"]
    kc, vc = case["kp"].copy(), case["vp"].copy()
    oracle.append(kc, oracle.project(case["x"], case["wk"]).reshape(B, T, Hkv, d), case["past_len"], dtype)
    oracle.append(vc, oracle.project(case["x"], case["wv"]).reshape(B, T, Hkv, d), case["past_len"], dtype)
    for b in range(B):
        L = int(case["past_len"][b])
        assert np.array_equal(kg[b, :, L:L + T], synth.to_storage(kc[b, :, L:L + T], dtype))
        assert np.array_equal(vg[b, :, L:L + T], synth.to_storage(vc[b, :, L:L + T], dtype))
        assert np.array_equal(kg[b, :, L + T:].view(np.uint8), before_k[b, :, L + T:].view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_append_random_values(dtype):
    case = _case(12, 2, 300, [17, 250], 512, 8, 2, 128, dtype)
    g = GpuLayer(case)
    try:
        g.append(case["x"], case["past_len"])
        kg, vg = g.cache_k(), g.cache_v()
    finally:
        g.free()
    import oracle
    B, T, Hkv, d = case["B"], case["T"], case["Hkv"], case["d"]
    kc, vc = case["kp"].copy(), case["vp"].copy()
    oracle.append(kc, oracle.project(case["x"], case["wk"]).reshape(B, T, Hkv, d), case["past_len"], dtype)
    oracle.append(vc, oracle.project(case["x"], case["wv"]).reshape(B, T, Hkv, d), case["past_len"], dtype)
    D = case["D"]
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in range(B):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L:L + T], kc[b, :, L:L + T], dtype, ak[b], D, "K rows")
        compare_rows(vg[b, :, L:L + T], vc[b, :, L:L + T], dtype, av[b], D, "V rows")


# ------------------------------------------------------------------ decode

DECODE_CASES = [
    # B, past, D, Hq, Hkv, d, dtype
    (1, [0], 256, 4, 4, 64, "f32"),
    (1, [300], 256, 4, 4, 64, "f32"),
    (3, [0, 1, 1000], 256, 8, 2, 128, "bf16"),
    (2, [777, 5000], 512, 16, 2, 64, "f16"),
    (2, [2000, 3001], 512, 16, 2, 128, "bf16"),   # G = 8
    (4, [64, 4095, 4096, 12345], 512, 8, 4, 128, "bf16"),
    (2, [1500, 999], 256, 4, 2, 128, "f32"),
]


@pytest.mark.parametrize("shape", DECODE_CASES, ids=lambda s: f"B{s[0]}-L{max(s[1])}-G{s[3]//s[4]}-d{s[5]}-{s[6]}")
def test_decode_parity(shape):
    B, past, D, Hq, Hkv, d, dtype = shape
    case = _case(13, B, 1, past, D, Hq, Hkv, d, dtype)
    g = GpuLayer(case, canary=True)
    try:
        before = g.cache.k.copy()
        out = g.decode(case["x"], case["past_len"])
        kg, vg = g.cache_k(), g.cache_v()
        after = g.cache.k
        for b in range(B):
            L = int(case["past_len"][b])
            assert np.array_equal(after[b, :, :L].view(np.uint8), before[b, :, :L].view(np.uint8))
            assert np.array_equal(after[b, :, L + 1:].view(np.uint8), before[b, :, L + 1:].view(np.uint8))
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(out, ref, dtype, f"decode {shape}")
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in range(B):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L], kc[b, :, L], dtype, ak[b, :, 0], D, "new K row")
        compare_rows(vg[b, :, L], vc[b, :, L], dtype, av[b, :, 0], D, "new V row")


@pytest.mark.parametrize("shape", [(2, [2000, 3001], 512, 16, 2, 128, "bf16"), (3, [0, 1, 700], 256, 4, 4, 64, "f32"),
                                   (1, [9000], 1024, 32, 8, 128, "f16")],
                         ids=lambda s: f"B{s[0]}-L{max(s[1])}-G{s[3]//s[4]}-{s[6]}")
def test_decode_query_prepass_is_bitwise_the_in_kernel_projection(shape, monkeypatch):
    """Queries projected once per step by the pre-pass and queries projected by each decode
    workgroup follow one summation order: the outputs and appended rows are bitwise equal."""
    B, past, D, Hq, Hkv, d, dtype = shape
    case = _case(17, B, 1, past, D, Hq, Hkv, d, dtype)
    outs, rows = [], []
    for mode in ("1", "0"):
        monkeypatch.setenv("DIRECTKV_DECODE_QPASS", mode)
        g = GpuLayer(case)
        try:
            outs.append(g.decode(case["x"], case["past_len"]))
            rows.append([(g.cache.k[b, :, L].copy(), g.cache.v[b, :, L].copy())
                         for b, L in enumerate(case["past_len"])])
        finally:
            g.free()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    for (k1, v1), (k0, v0) in zip(rows[0], rows[1]):
        assert np.array_equal(k1.view(np.uint8), k0.view(np.uint8))
        assert np.array_equal(v1.view(np.uint8), v0.view(np.uint8))
    kc, vc = case["kp"].copy(), case["vp"].copy()
    compare(outs[0], oracle_step(case, case["x"], case["past_len"], kc, vc), dtype, f"decode {shape}")


@pytest.mark.parametrize("shape", [(1, [0], 256, 4, 4, 64, "f32"), (4, [0, 5, 100, 120], 256, 16, 4, 128, "bf16"),
                                   (2, [63, 64], 512, 16, 2, 128, "f16")],
                         ids=lambda s: f"B{s[0]}-L{max(s[1])}-G{s[3]//s[4]}-{s[6]}")
def test_single_split_decode_writes_the_output_directly(shape, monkeypatch):
    """With one split per sequence the decode kernel writes the output itself (no combine
    launch): bitwise what the combine gives from the same partials, and within the tolerance of
    the oracle."""
    B, past, D, Hq, Hkv, d, dtype = shape
    case = _case(29, B, 1, past, D, Hq, Hkv, d, dtype)
    outs = []
    for mode in ("0", "1"):
        monkeypatch.setenv("DIRECTKV_DECODE_COMBINE", mode)
        g = GpuLayer(case)
        try:
            outs.append(g.decode(case["x"], case["past_len"]))
        finally:
            g.free()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    kc, vc = case["kp"].copy(), case["vp"].copy()
    compare(outs[0], oracle_step(case, case["x"], case["past_len"], kc, vc), dtype, f"decode {shape}")


def test_decode_at_the_batch_limit(monkeypatch):
    """256 sequences (the most one call takes) with ragged lengths from 0 up: one to three
    splits each, the split table's last entries, and the query pre-pass's 32 grid rows of 8
    sequences. Both query paths against the oracle, and bitwise against each other."""
    B, D, Hq, Hkv, d, dtype = 256, 128, 8, 2, 64, "bf16"
    past = [int(v) for v in synth.Draw(23).lengths(B, 0, 300)]
    past[0], past[-1] = 0, 300
    case = _case(23, B, 1, past, D, Hq, Hkv, d, dtype)
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    outs = []
    for mode in ("1", "0"):
        monkeypatch.setenv("DIRECTKV_DECODE_QPASS", mode)
        g = GpuLayer(case)
        try:
            outs.append(g.decode(case["x"], case["past_len"]))
            kg = g.cache_k()
        finally:
            g.free()
        compare(outs[-1], ref, dtype, f"decode B=256 qpass={mode}")
        ak = absdot_rows(case["x"], case["wk"], Hkv, d)
        for b in (0, 1, 127, 255):
            L = int(case["past_len"][b])
            compare_rows(kg[b, :, L], kc[b, :, L], dtype, ak[b, :, 0], D, f"new K row of sequence {b}")
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


# ------------------------------------------------------------------ prefill


@pytest.mark.parametrize("two_launch", ["1", "0"], ids=["two-launch", "per-chunk"])
def test_prefill_at_the_batch_limit(two_launch, monkeypatch):
    """256 sequences (the most one call takes), ragged pasts from 0 to 300, 2 query tiles per
    (sequence, kv head) pair (512 pairs), 64-key super-chunks: up to 5 of them per sequence,
    empty ones for the short pasts. Sampled rows against the oracle; the appended rows of the first,
    middle and last sequences within the accumulation bound."""
    monkeypatch.setenv("DIRECTKV_PREFILL_CHUNKED", two_launch)
    monkeypatch.setenv("DIRECTKV_PREFILL_CHUNK", "64")
    B, T, D, Hq, Hkv, d, dtype = 256, 40, 128, 16, 2, 64, "bf16"
    past = [int(v) for v in synth.Draw(24).lengths(B, 0, 300)]
    past[0], past[1], past[-1] = 0, 64, 300
    case = _case(24, B, T, past, D, Hq, Hkv, d, dtype)
    ts = np.array([0, 1, 19, 38, 39])
    out, ref, kg, vg, kc, vc = _run_prefill(case, t_index=ts)
    compare(out, ref, dtype, f"prefill B=256 two_launch={two_launch}")
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in (0, 1, 128, 255):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L:L + T], kc[b, :, L:L + T], dtype, ak[b], D, f"new K rows of sequence {b}")
        compare_rows(vg[b, :, L:L + T], vc[b, :, L:L + T], dtype, av[b], D, f"new V rows of sequence {b}")

PREFILL_CASES = [
    # B, T, past, D, Hq, Hkv, d, dtype
    (1, 128, [0], 256, 4, 4, 64, "f32"),             # the tiny fp32 layer
    (2, 200, [100, 300], 512, 8, 2, 128, "bf16"),
    (2, 77, [0, 1029], 256, 16, 2, 64, "f16"),       # G = 8, ragged tail
    (1, 300, [5000], 256, 4, 1, 128, "bf16"),        # two key super-chunks
    (2, 300, [3000, 4500], 512, 32, 8, 128, "bf16"),  # 16 pairs: two groups of 8, super-chunks each
    (1, 130, [70], 256, 8, 4, 128, "f32"),
    (3, 150, [900, 0, 2500], 256, 16, 8, 64, "f16"),  # 24 pairs: three groups of 8
    (3, 100, [500, 0, 2200], 256, 8, 4, 64, "bf16"),  # 12 pairs: one launch group, 2 pairs per XCD
    (1, 70, [33], 192, 4, 2, 64, "bf16"),            # 3 projection reduction steps (odd tail)
    (2, 20, [0, 45], 320, 8, 8, 128, "f16"),         # 5 reduction steps; one key tile for b = 0
    (1, 1, [0], 256, 4, 4, 64, "f32"),               # one token on an empty cache: its own V
    (3, 1, [1000, 0, 63], 256, 16, 2, 128, "bf16"),  # one token per sequence, ragged pasts
    (2, 1, [64, 4096], 256, 32, 8, 128, "f16"),      # one token after a whole tile / super-chunk
]


@pytest.mark.parametrize("shape", PREFILL_CASES, ids=lambda s: f"B{s[0]}-T{s[1]}-L{max(s[2])}-G{s[4]//s[5]}-d{s[6]}-{s[7]}")
def test_prefill_parity(shape):
    B, T, past, D, Hq, Hkv, d, dtype = shape
    case = _case(14, B, T, past, D, Hq, Hkv, d, dtype)
    out, ref, kg, vg, kc, vc = _run_prefill(case, canary=True)
    compare(out, ref, dtype, f"prefill {shape}")
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in range(B):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L:L + T], kc[b, :, L:L + T], dtype, ak[b], D, "new K rows")
        compare_rows(vg[b, :, L:L + T], vc[b, :, L:L + T], dtype, av[b], D, "new V rows")


def test_prefill_long_launch_super_chunks_sampled_rows():
    """257 query tiles of 256 rows for the one (sequence, kv head) pair: the planner takes the
    smaller super-chunk it uses for launches with many rounds of query tiles (3072 keys at bf16,
    d = 128), whose boundaries fall inside the past and inside the new keys. Sampled token rows
    (every head) against the oracle, and every appended row."""
    B, T, past, D, Hq, Hkv, d, dtype = 1, 8200, [2000], 256, 8, 1, 128, "bf16"
    ts = np.array(sorted({0, 1, 1071, 1072, 3000, 4095, 4096, 7167, 7168, 8191, 8198, 8199}))
    case = _case(19, B, T, past, D, Hq, Hkv, d, dtype)
    out, ref, kg, vg, kc, vc = _run_prefill(case, t_index=ts, canary=True)
    compare(out, ref, dtype, "long-launch prefill, sampled rows")
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    L = past[0]
    compare_rows(kg[0, :, L:L + T], kc[0, :, L:L + T], dtype, ak[0], D, "new K rows")
    compare_rows(vg[0, :, L:L + T], vc[0, :, L:L + T], dtype, av[0], D, "new V rows")


def test_tiny_layer_prefill_then_decode():
    """The tiny fp32 layer: causal prefill of 128 tokens into an empty cache, then one
    decode step reading the cache the prefill wrote."""
    w = synth.WORKLOADS[0]
    case = synth.draw_layer(w.seed, w.B, w.T, w.past, w.D, w.Hq, w.Hkv, w.d, w.dtype, w.cap)
    xdec = synth.Draw(w.seed + 500).normal((w.B, 1, w.D), 1.0, w.dtype)
    g = GpuLayer(case)
    try:
        out_p = g.prefill(case["x"], case["past_len"])
        out_d = g.decode(xdec, case["past_len"] + w.T)
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref_p = oracle_step(case, case["x"], case["past_len"], kc, vc)
    ref_d = oracle_step(case, xdec, case["past_len"] + w.T, kc, vc)
    compare(out_p, ref_p, "f32", "tiny prefill")
    compare(out_d, ref_d, "f32", "tiny decode")


def test_prefill_key_splits_ragged_with_empty_splits():
    """One query tile per pair (T * G <= 256): each pair's keys are split over workgroups and a
    second launch merges the splits. With a long and an empty past in one call, the short pair
    has fewer key tiles than splits, so most of its splits (the first among them) see no keys."""
    case = _case(21, 3, 16, [0, 9000, 130], 256, 16, 2, 128, "bf16")
    out, ref, kg, vg, kc, vc = _run_prefill(case, canary=True)
    compare(out, ref, "bf16", "prefill with key splits")
    ak = absdot_rows(case["x"], case["wk"], case["Hkv"], case["d"])
    av = absdot_rows(case["x"], case["wv"], case["Hkv"], case["d"])
    for b in range(case["B"]):
        L = int(case["past_len"][b])
        compare_rows(kg[b, :, L:L + 16], kc[b, :, L:L + 16], "bf16", ak[b], case["D"], "new K rows")
        compare_rows(vg[b, :, L:L + 16], vc[b, :, L:L + 16], "bf16", av[b], case["D"], "new V rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_token_prefill_matches_decode(dtype):
    """A prefill of one token (key splits over the whole cache) against the decode step on the
    same inputs and the oracle."""
    case = _case(22, 2, 1, [5000, 777], 256, 8, 2, 128, dtype)
    g = GpuLayer(case)
    try:
        p = g.prefill(case["x"], case["past_len"])
    finally:
        g.free()
    g = GpuLayer(case)
    try:
        dcd = g.decode(case["x"], case["past_len"])
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc)
    compare(p, ref, dtype, "one-token prefill")
    compare(dcd, ref, dtype, "decode")


# ------------------------------------------------------------------ invariants

def test_prefill_causal_perturbation_is_bitwise():
    case = _case(15, 1, 160, [200], 256, 8, 2, 128, "bf16")
    g = GpuLayer(case)
    try:
        a = g.prefill(case["x"], case["past_len"])
        x2 = case["x"].copy()
        x2[:, 100:] = synth.Draw(99).normal(x2[:, 100:].shape, 1.0, "bf16")
        b = g.prefill(x2, case["past_len"])
    finally:
        g.free()
    assert np.array_equal(a[:, :100], b[:, :100])
    assert not np.array_equal(a[:, 100:], b[:, 100:])


def test_reruns_are_bit_identical():
    case = _case(16, 2, 1, [3000, 777], 512, 8, 2, 128, "bf16")
    g = GpuLayer(case)
    try:
        d1 = g.decode(case["x"], case["past_len"])
        d2 = g.decode(case["x"], case["past_len"])
        casep = _case(17, 1, 200, [1000], 256, 8, 2, 128, "bf16")
    finally:
        g.free()
    assert np.array_equal(d1, d2)
    gp = GpuLayer(casep)
    try:
        p1 = gp.prefill(casep["x"], casep["past_len"])
        p2 = gp.prefill(casep["x"], casep["past_len"])
    finally:
        gp.free()
    assert np.array_equal(p1, p2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_phase_consistency(dtype):
    """prefill(T) ~ prefill(T1) + prefill(T - T1) ~ T decode steps (same cache rows)."""
    T = 40
    case = _case(18, 2, T, [300, 65], 256, 8, 2, 128, dtype)
    past = case["past_len"]
    g1 = GpuLayer(case)
    try:
        whole = g1.prefill(case["x"], past)
    finally:
        g1.free()
    g2 = GpuLayer(case)
    try:
        a = g2.prefill(case["x"][:, :15], past)
        b = g2.prefill(case["x"][:, 15:], past + 15)
    finally:
        g2.free()
    g3 = GpuLayer(case)
    try:
        steps = [g3.decode(case["x"][:, t:t + 1], past + t) for t in range(T)]
    finally:
        g3.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], past, kc, vc)
    compare(whole, ref, dtype, "whole")
    compare(np.concatenate([a, b], axis=1), ref, dtype, "two chunks")
    compare(np.concatenate(steps, axis=1), ref, dtype, "decode steps")


def test_constant_values_give_the_constant():
    """Wv passes X column 0 (set to 1) scaled by c, past V = c: every output is c."""
    case = _case(19, 2, 50, [100, 900], 256, 8, 2, 128, "bf16")
    c = 0.375
    case["wv"][:] = 0.0
    case["wv"][0, :] = c
    case["x"][:, :, 0] = 1.0
    case["vp"][:] = c
    g = GpuLayer(case)
    try:
        out = g.prefill(case["x"], case["past_len"])
        outd = g.decode(case["x"][:, :1], case["past_len"] + 50)
    finally:
        g.free()
    assert np.all(np.abs(out - c) <= 2e-3)
    assert np.all(np.abs(outd - c) <= 2e-3)


def test_host_cache_allocates_no_device_memory():
    import torch
    import zero_copy_host_amd as dkv
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    free_before, _ = torch.cuda.mem_get_info()
    cache = dkv.HostKVCache(4, 8, 128, 65536, "bf16")   # 1 GiB of K + V
    cache.k[0, 0, :4] = 1
    free_after, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == before
    assert free_before - free_after < cache.nbytes() // 8
    cache.free()


def test_rejected_calls_enqueue_nothing_and_touch_nothing():
    import torch
    import zero_copy_host_amd as dkv
    case = _case(20, 2, 4, [10, 20], 256, 8, 2, 128, "bf16", cap=64)
    g = GpuLayer(case, canary=True)
    try:
        before = g.cache.k.copy()
        with pytest.raises(dkv.DirectKVError) as e:
            g.prefill(np.zeros((2, 60, 256), np.float32), case["past_len"])   # 20 + 60 > 64
        assert e.value.status == -2
        ws = torch.empty(16, dtype=torch.uint8, device="cuda")
        out = torch.empty((2, 1, 8 * 128), dtype=torch.bfloat16, device="cuda")
        x = torch.zeros((2, 1, 256), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(dkv.DirectKVError) as e:
            dkv.attn_decode(g.cache, x, g.wq, g.wk, g.wv, case["past_len"], 8, out, ws)
        assert e.value.status == -6
        torch.cuda.synchronize()
        assert np.array_equal(g.cache.k.view(np.uint8), before.view(np.uint8))
    finally:
        g.free()


@pytest.mark.parametrize("variant", ["naive", "separate"])
def test_prefill_ablation_variants_match_the_oracle(variant):
    """The baselines the pages compare against compute the same layer step."""
    import torch
    from gpu_case import to_dev, torch_dtype
    case = _case(21, 2, 300, [3000, 4500], 512, 32, 8, 128, "bf16")
    g = GpuLayer(case, canary=True)
    try:
        B, T = case["B"], case["T"]
        out = torch.empty((B, T, case["Hq"] * case["d"]), dtype=torch_dtype("bf16"), device="cuda")
        ws = torch.empty(g.dkv.workspace_bytes("prefill", g.cache, B, T, case["Hq"]), dtype=torch.uint8, device="cuda")
        g.dkv.attn_prefill_variant(g.cache, to_dev(case["x"], "bf16"), g.wq, g.wk, g.wv, case["past_len"],
                                   case["Hq"], out, ws, variant)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().reshape(B, T, case["Hq"], case["d"])
    finally:
        g.free()
    ref = oracle_step(case, case["x"], case["past_len"], case["kp"].copy(), case["vp"].copy())
    compare(got, ref, "bf16", f"prefill variant {variant}")
