"""Rotary position embedding on the GPU (attn_prefill_rope, attn_decode_rope) against the oracle,
through the C ABI.

q and the new k are rotated at positions past_len[b] + t before the attention and before k is
rounded and appended, with pair (i, i + d/2) of a head turned by p * theta^(-2i/d). The GPU forms
the angles in fp64 and rotates the fp32 projections with fp32 (cos, sin); the oracle rotates in
fp64. The attention outputs are held to the layer's tolerances (max-abs 2e-2 / mean-abs 2e-3 for
bf16 and f16, 1e-5 for fp32). The appended K rows are held to the rotated fp32-accumulation bound:
each of the two rotated terms carries its projection's D * 2^-24 * sum|x||w| error, the fp32
table values and products add a few 2^-24 of |k_lo| + |k_hi|, and the one rounding to the cache
dtype adds at most an ulp. V rows are not rotated and keep the plain bound."""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import GpuLayer, _ulp, absdot_rows, compare, compare_rows, oracle_step

pytestmark = pytest.mark.gpu


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype):
    cap = ((max(past) + T + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap)


def _rotated_rows_bound(case, d):
    """Bound on |GPU - oracle| for rotated new K rows, [B, Hkv, T, d]."""
    B, T, D, Hkv = case["B"], case["T"], case["D"], case["Hkv"]
    ak = absdot_rows(case["x"], case["wk"], Hkv, d)        # sum|x||w| per element, >= |k|
    half = d // 2
    pair = np.concatenate([ak[..., :half] + ak[..., half:]] * 2, axis=-1)   # both terms of a rotated element
    return (D + 4) * 2.0 ** -24 * pair


def _check_rope_rows(kg, vg, kc, vc, case, what):
    B, T, D, Hkv, d, dtype = case["B"], case["T"], case["D"], case["Hkv"], case["d"], case["dtype"]
    bound = _rotated_rows_bound(case, d)
    av = absdot_rows(case["x"], case["wv"], Hkv, d)
    for b in range(B):
        L = int(case["past_len"][b])
        ref = kc[b, :, L:L + T].astype(np.float64)
        err = np.abs(kg[b, :, L:L + T] - ref)
        bad = err > bound[b] + _ulp(ref, dtype)
        assert not bad.any(), f"{what}: {int(bad.sum())} rotated K values outside the bound"
        compare_rows(vg[b, :, L:L + T], vc[b, :, L:L + T], dtype, av[b], D, f"{what}: V rows")


PREFILL = [
    # B, T, past, D, Hq, Hkv, d, dtype, rope base
    (1, 200, [3000], 256, 8, 2, 128, "bf16", 500000.0),
    (2, 100, [500, 1700], 256, 16, 2, 64, "f16", 10000.0),
    (1, 97, [1000], 256, 8, 2, 128, "f32", 500000.0),
    (3, 64, [0, 300, 2100], 256, 8, 2, 128, "bf16", 10000.0),
    (1, 300, [20], 256, 8, 8, 64, "f32", 10000.0),
]


def _ids(s):
    return f"B{s[0]}-T{s[1]}-L{max(s[2])}-G{s[4] // s[5]}-d{s[6]}-{s[7]}-th{int(s[8])}"


@pytest.mark.parametrize("shape", PREFILL, ids=_ids)
def test_prefill_rope_parity(shape):
    B, T, past, D, Hq, Hkv, d, dtype, theta = shape
    case = _case(601, B, T, past, D, Hq, Hkv, d, dtype)
    print(f"prefill rope {_ids(shape)}", flush=True)
    g = GpuLayer(case)
    try:
        out = g.prefill(case["x"], case["past_len"], rope_theta=theta)
        kg, vg = g.cache_k(), g.cache_v()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc, rope_theta=theta)
    compare(out, ref, dtype, f"prefill rope {_ids(shape)}")
    _check_rope_rows(kg, vg, kc, vc, case, "prefill rope")
    # the rotation is not a no-op here: the unrotated layer gives another answer
    kc0, vc0 = case["kp"].copy(), case["vp"].copy()
    ref0 = oracle_step(case, case["x"], case["past_len"], kc0, vc0)
    assert np.abs(ref0 - ref).max() > 10 * max(1e-5, np.abs(out - ref).max())


def test_prefill_rope_far_positions_sampled_rows():
    """Positions near 100000, where the fastest pair's angle passes 10^5 radians: sampled token
    rows against the oracle, every rotated K row against the bound."""
    B, T, past, D, Hq, Hkv, d, dtype, theta = 1, 300, [99800], 256, 8, 2, 128, "bf16", 500000.0
    case = _case(602, B, T, past, D, Hq, Hkv, d, dtype)
    ts = np.array([0, 1, 150, 255, 256, 299])
    g = GpuLayer(case)
    try:
        out = g.prefill(case["x"], case["past_len"], rope_theta=theta)
        kg, vg = g.cache_k(), g.cache_v()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc, t_index=ts, rope_theta=theta)
    compare(out[:, ts], ref, dtype, "prefill rope far positions")
    _check_rope_rows(kg, vg, kc, vc, case, "prefill rope far positions")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_rope_parity(dtype):
    """Ragged decode (one, several and many splits per sequence) at positions up to 70000."""
    case = _case(603, 3, 1, [37, 5000, 70000], 256, 8, 2, 128, dtype)
    theta = 500000.0
    g = GpuLayer(case)
    try:
        out = g.decode(case["x"], case["past_len"], rope_theta=theta)
        kg, vg = g.cache_k(), g.cache_v()
    finally:
        g.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], case["past_len"], kc, vc, rope_theta=theta)
    compare(out, ref, dtype, f"decode rope {dtype}")
    _check_rope_rows(kg, vg, kc, vc, case, f"decode rope {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_phase_consistency(dtype):
    """With RoPE, prefill(T) ~ prefill(T1) + prefill(T - T1) ~ T decode steps: every path
    rotates at the same absolute positions."""
    T, theta = 40, 10000.0
    case = _case(604, 2, T, [300, 65], 256, 8, 2, 64, dtype)
    past = case["past_len"]
    g1 = GpuLayer(case)
    try:
        whole = g1.prefill(case["x"], past, rope_theta=theta)
    finally:
        g1.free()
    g2 = GpuLayer(case)
    try:
        a = g2.prefill(case["x"][:, :15], past, rope_theta=theta)
        b = g2.prefill(case["x"][:, 15:], past + 15, rope_theta=theta)
    finally:
        g2.free()
    g3 = GpuLayer(case)
    try:
        steps = [g3.decode(case["x"][:, t:t + 1], past + t, rope_theta=theta) for t in range(T)]
    finally:
        g3.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, case["x"], past, kc, vc, rope_theta=theta)
    compare(whole, ref, dtype, "whole")
    compare(np.concatenate([a, b], axis=1), ref, dtype, "two chunks")
    compare(np.concatenate(steps, axis=1), ref, dtype, "decode steps")
