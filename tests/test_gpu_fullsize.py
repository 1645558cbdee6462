"""Parity at the full sizes of the named workloads, in the launch configuration the benchmark
uses. Decode outputs are compared in full; prefill outputs on sampled token rows (every
head), which the oracle computes after projecting and appending every new row. The sampled
rows include the rows on each side of every 1024-key boundary of the keys a row sees (launch
ranges and key tiles are multiples of 64 keys), and the appended cache rows of the sampled
tokens are compared against the oracle's within the fp32-accumulation bound."""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import GpuLayer, absdot_rows, compare, compare_rows

pytestmark = pytest.mark.gpu


def _workload_case(name):
    w = synth.workload(name)
    case = synth.draw_layer(w.seed, w.B, w.T, w.past, w.D, w.Hq, w.Hkv, w.d, w.dtype, w.cap,
                            past_lo=w.past_lo, past_hi=w.past_hi)
    return w, case


def _sample_tokens(T, L=0, seed=0, n_random=8, stride=1024):
    """Fixed rows (first, last, tile edges), random rows, and for every multiple of `stride` keys
    the two query rows whose last visible key sits just below and at that boundary."""
    fixed = {0, 1, 63, 64, 127, 128, 255, 256, T // 2, T - 2, T - 1}
    for k in range((L // stride + 1) * stride, L + T + 1, stride):
        fixed |= {k - L - 1, k - L}          # row t sees keys 0 .. L + t
    rng = np.random.default_rng(seed)
    extra = set(int(x) for x in rng.integers(0, T, size=n_random))
    return np.array(sorted(t for t in fixed | extra if 0 <= t < T))


def _appended_rows(g, case, ts):
    """The host cache rows [L_b + t] of the sampled tokens, K and V, as float32 [B, Hkv, n, d]."""
    L = case["past_len"]
    # (index the sequence first: g.cache.k[b, :, rows] would put the sampled axis first)
    k = np.stack([synth.from_storage(g.cache.k[b][:, int(L[b]) + ts], case["dtype"]) for b in range(case["B"])])
    v = np.stack([synth.from_storage(g.cache.v[b][:, int(L[b]) + ts], case["dtype"]) for b in range(case["B"])])
    return k, v


def _check_appended(case, ts, kg, vg, kc, vc, what):
    L = case["past_len"]
    xs = case["x"][:, ts]
    ak = absdot_rows(xs, case["wk"], case["Hkv"], case["d"])
    av = absdot_rows(xs, case["wv"], case["Hkv"], case["d"])
    for b in range(case["B"]):
        rows = int(L[b]) + ts
        compare_rows(kg[b], kc[b][:, rows], case["dtype"], ak[b], case["D"], f"{what} K rows")
        compare_rows(vg[b], vc[b][:, rows], case["dtype"], av[b], case["D"], f"{what} V rows")


@pytest.mark.parametrize("name", ["llama8b_decode_b8_L32768_bf16", "long_decode_b4_L96k_128k_f16"])
def test_decode_full_size(name):
    w, case = _workload_case(name)
    print(f"{name}: past_len={case['past_len'].tolist()}", flush=True)
    g = GpuLayer(case)
    try:
        out = g.decode(case["x"], case["past_len"])
    finally:
        g.free()
    ref = oracle.layer_step(case["x"], case["wq"], case["wk"], case["wv"], case["kp"], case["vp"],
                            case["past_len"], w.Hq, w.dtype)
    compare(out, ref, w.dtype, name)


def test_prefill_full_size_llama8b_sampled_rows():
    w, case = _workload_case("llama8b_prefill_T8192_on_L24576_bf16")
    ts = _sample_tokens(w.T, int(case["past_len"][0]))
    g = GpuLayer(case)
    try:
        out = g.prefill(case["x"], case["past_len"])
        kg, vg = _appended_rows(g, case, ts)
    finally:
        g.free()
    ref = oracle.layer_step(case["x"], case["wq"], case["wk"], case["wv"], case["kp"], case["vp"],
                            case["past_len"], w.Hq, w.dtype, t_index=ts)
    compare(out[:, ts], ref, w.dtype, f"{w.name} rows {ts.tolist()}")
    _check_appended(case, ts, kg, vg, case["kp"], case["vp"], w.name)


def test_llama70b_prefill_then_decode_steps_sampled():
    """16384-token prefill on 49152 host-resident past tokens, batch 2, then 64 decode
    steps; prefill rows and decode steps are sampled, every step is appended by both."""
    w, case = _workload_case("llama70b_prefill_T16384_on_L49152_b2_bf16")
    steps = w.decode_steps
    dr = synth.Draw(w.seed + 1)
    xs = [dr.normal((w.B, 1, w.D), 1.0, w.dtype) for _ in range(steps)]
    check_steps = {0, 1, steps // 2, steps - 1}
    ts = _sample_tokens(w.T, int(case["past_len"][0]), seed=1, stride=2048)
    g = GpuLayer(case)
    outs = []
    try:
        out_p = g.prefill(case["x"], case["past_len"])
        kg, vg = _appended_rows(g, case, ts)
        for s in range(steps):
            outs.append(g.decode(xs[s], case["past_len"] + w.T + s))
    finally:
        g.free()
    kc, vc = case["kp"], case["vp"]
    ref = oracle.layer_step(case["x"], case["wq"], case["wk"], case["wv"], kc, vc,
                            case["past_len"], w.Hq, w.dtype, t_index=ts)
    compare(out_p[:, ts], ref, w.dtype, f"{w.name} prefill rows {ts.tolist()}")
    _check_appended(case, ts, kg, vg, kc, vc, f"{w.name} prefill")
    for s in range(steps):
        sel = [0] if s in check_steps else []
        refd = oracle.layer_step(xs[s], case["wq"], case["wk"], case["wv"], kc, vc,
                                 case["past_len"] + w.T + s, w.Hq, w.dtype, t_index=sel)
        if sel:
            compare(outs[s], refd, w.dtype, f"{w.name} decode step {s}")
