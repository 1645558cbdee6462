"""Benchmark of the host-KV attention layer on one MI355X.

Headline workload: the Llama-3-70B-shaped layer in bf16 (D=8192, Hq=64, Hkv=8, d=128), batch 2:
a chunked prefill of 16384 new tokens per sequence on 49152 past tokens held in pinned host
memory (the cache then holds 65536 tokens), followed by 64 decode steps over that cache. A timed
step is one attn_prefill call: the Q/K/V projection of the new tokens, their append to the host
cache, and causal grouped-query attention over every past and new key; the value is prefill
tokens per second (B*T / step time), and the 64 decode steps after it are reported beside it in
microseconds per step. Inputs are synthetic (seeded N(0,1) activations and past K/V, N(0, 1/D)
weights) and resident before timing starts: X and W in device memory, the KV cache in pinned host
memory, where the method keeps it.

Prints one JSON line. Extra objects: the measured host-link peak (kernel streaming read/write of
pinned memory), the roofline of the dominant kernel (prefill attention: its duration from HIP
events on the library's stream, its algorithmic flops per launch), the oracle timed on the host
cores over a bounded sample (cpu_baseline), and every other named workload (8B-shaped decode and
chunked prefill, fp16 long-context decode, the tiny fp32 layer, ablations, paged cache, staging
baseline, decoder stack) each with its own roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 63.0      # published PCIe 5.0 x16 rate per direction (32 GT/s, 128b/130b)
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def tdtype(dt):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_dev(a, dt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdtype(dt)).cuda()


class EventTimer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.s.record()
        return self

    def __exit__(self, *a):
        self.e.record()
        self.e.synchronize()
        self.ms = self.s.elapsed_time(self.e)


def _timed_phases(dkv, fn, n):
    """Run fn() n times with the library's per-phase kernel timing on; returns its records."""
    import torch
    torch.cuda.synchronize()
    dkv.timing(True)
    try:
        for _ in range(n):
            fn()
        return dkv.timing_read()
    finally:
        dkv.timing(False)


def hostlink_peak(dkv, nbytes=1 << 30, reps=8):
    """Kernel streaming read and write rate of pinned host memory (GB/s): the best of `reps`
    separately timed passes over a 1 GiB buffer (a peak, so one slow pass does not lower it)."""
    import torch
    cap = nbytes // (128 * 2)
    buf = dkv.HostKVCache(1, 1, 128, cap, "bf16")
    ptr = buf.desc.k
    res = {}
    for mode in ("read", "write"):
        dkv.hostlink_stream(ptr, nbytes, mode, 1024)
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(reps):
            with EventTimer() as t:
                dkv.hostlink_stream(ptr, nbytes, mode, 1024)
            best = max(best, nbytes / (t.ms * 1e-3) / 1e9)
        res[mode] = best
    buf.free()
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads():
    """Threads for the C oracle: the host cores this process may use, at most 16 (a one-GPU machine's
    share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_prefill(name, n_tokens=384):
    """The oracle, as it is, on a bounded sample of workload `name`'s prefill step: the first
    n_tokens of the step's new tokens (every sequence, every head), on the same past keys, timed
    in the oracle's threaded C form (fp64 loops over (sequence, kv head, block of query tokens)).
    Its rate is the sample's tokens over the oracle's time; later tokens of the full step see up
    to T more keys, so the full step would run slower per token."""
    from oracle import cref
    import synth
    w = synth.workload(name)
    dr = synth.Draw(w.seed)
    wq, wk, wv = synth.layer_weights(dr, w.D, w.Hq, w.Hkv, w.d, w.dtype)
    past = np.asarray(w.past, dtype=np.int32) if w.past is not None else dr.lengths(w.B, w.past_lo, w.past_hi)
    x = dr.normal((w.B, w.T, w.D), 1.0, w.dtype)[:, :n_tokens]
    cap = int(max(past)) + n_tokens
    kc = np.zeros((w.B, w.Hkv, cap, w.d), dtype=np.float32)
    vc = np.zeros_like(kc)
    synth.fill_past(dr, kc, vc, past, w.dtype)
    threads = _oracle_threads()
    cref.lib()
    t0 = time.perf_counter()
    cref.layer_step(x, wq, wk, wv, kc, vc, past, w.Hq, w.dtype, threads=threads)
    el = time.perf_counter() - t0
    tok = w.B * n_tokens
    return {"value": tok / el, "unit": "prefill tok/s per layer", "cores": threads, "kind": "oracle",
            "seconds": el, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"the first {n_tokens} of the {w.T} new tokens of each of the {w.B} sequences of {name} "
                      f"(projection, append, causal attention over {int(past[0])}+ keys, all {w.Hq} heads), "
                      f"fp64 C oracle on {threads} threads; the full step's later tokens see up to {w.T} more "
                      f"keys each"}


def cpu_baseline_decode(name, min_seconds=10.0):
    """The oracle, as it is, on whole decode steps of workload `name`, repeated for ~min_seconds,
    in its threaded C form."""
    from oracle import cref
    import synth
    w = synth.workload(name)
    dr = synth.Draw(w.seed)
    wq, wk, wv = synth.layer_weights(dr, w.D, w.Hq, w.Hkv, w.d, w.dtype)
    past = np.asarray(w.past, dtype=np.int32) if w.past is not None else dr.lengths(w.B, w.past_lo, w.past_hi)
    x = dr.normal((w.B, 1, w.D), 1.0, w.dtype)
    kc = np.zeros((w.B, w.Hkv, w.cap, w.d), dtype=np.float32)
    vc = np.zeros_like(kc)
    synth.fill_past(dr, kc, vc, past, w.dtype)
    threads = _oracle_threads()
    cref.lib()
    t0 = time.perf_counter()
    n = 0
    while True:
        cref.layer_step(x, wq, wk, wv, kc, vc, past, w.Hq, w.dtype, threads=threads)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": el / n * 1e6, "unit": "us per layer decode step", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{n} full decode step(s) of {name} (all {w.B} sequences, {int(past[0]) + 1} keys each), "
                      f"fp64 C oracle on {threads} threads"}


def read_counter_summary(name, kernel_src_hash):
    """Key/value lines of profiles/<name>_counters.txt if it was taken on the current kernel
    source (its kernel_source_sha1 line), else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha1") != kernel_src_hash:
        return None
    return vals


def _float(vals, key):
    try:
        return float(vals[key]) if vals else None
    except (KeyError, ValueError):
        return None


def src_hash(*names):
    h = hashlib.sha1()
    for n in names:
        h.update(open(os.path.join(ROOT, "zero_copy_host_amd", "csrc", n), "rb").read())
    return h.hexdigest()


def _layer_setup(dkv, w, seed_extra=0):
    """Weights, lengths, X of the first step and the filled host cache for workload w."""
    import synth
    dr = synth.Draw(w.seed + seed_extra)
    wq, wk, wv = synth.layer_weights(dr, w.D, w.Hq, w.Hkv, w.d, w.dtype)
    past = np.asarray(w.past, dtype=np.int32) if w.past is not None else dr.lengths(w.B, w.past_lo, w.past_hi)
    x = dr.normal((w.B, w.T, w.D), 1.0, w.dtype)
    cache = dkv.HostKVCache(w.B, w.Hkv, w.d, w.cap, w.dtype)
    synth.fill_past(dr, cache.k, cache.v, past, w.dtype)
    dev = dict(x=to_dev(x, w.dtype), wq=to_dev(wq.T, w.dtype), wk=to_dev(wk.T, w.dtype), wv=to_dev(wv.T, w.dtype))
    return past, cache, dev, dr


KEY_TILE = 64   # keys per tile of one (sequence, kv head) stream in both attention kernels


def _overlap_model(new_tokens, past, host_read, flops, peak_tflops, ms, peak_read):
    """The pages' two-stage pipeline model of the step as an expected time: the longest
    (sequence, kv head) key stream in 64-key tiles, its transfer at the measured link read peak
    and its compute at the dtype's dense MFMA peak."""
    from zero_copy_host_amd import accounting as acc
    if not peak_read:
        return None
    n_tiles = -(-(int(np.max(past)) + new_tokens) // KEY_TILE)
    expected = acc.overlap_model_seconds(n_tiles, host_read, flops, peak_read * 1e9, peak_tflops * 1e12) * 1e3
    return {"expected_ms": expected, "n_tiles": n_tiles, "link_GBps": peak_read, "compute_tflops": peak_tflops,
            "measured_over_expected": ms / expected if expected else None}


def _prefill_stats(w, past, ms, peak_read):
    import synth
    from zero_copy_host_amd import accounting as acc
    e = synth.elem_bytes(w.dtype)
    host_read = acc.host_read_bytes(past, w.Hkv, w.d, e)
    host_write = acc.host_write_bytes(w.B, w.T, w.Hkv, w.d, e)
    flops = acc.attention_flops(past, w.T, w.Hq, w.d) + acc.projection_flops(w.B, w.T, w.D, w.Hq, w.Hkv, w.d)
    mfma_peak = MFMA_PEAK_TFLOPS[w.dtype]
    tflops = flops / (ms * 1e-3) / 1e12
    return {"ms_per_step": ms, "tok_per_s": w.B * w.T / (ms * 1e-3),
            "tflops": tflops, "mfma_peak_tflops": mfma_peak, "mfma_frac": tflops / mfma_peak,
            "host_read_bytes": host_read, "host_write_bytes": host_write,
            "host_read_floor_ms": host_read / (peak_read * 1e9) * 1e3 if peak_read else None,
            "mfma_floor_ms": flops / (mfma_peak * 1e12) * 1e3,
            "overlap_model": _overlap_model(w.T, past, host_read, flops, mfma_peak, ms, peak_read)}


def _decode_stats(w, past, ms, peak_read):
    import synth
    from zero_copy_host_amd import accounting as acc
    e = synth.elem_bytes(w.dtype)
    host_read = acc.host_read_bytes(past, w.Hkv, w.d, e)
    gbps = host_read / (ms * 1e-3) / 1e9
    flops = acc.attention_flops(past, 1, w.Hq, w.d) + acc.projection_flops(w.B, 1, w.D, w.Hq, w.Hkv, w.d)
    return {"us_per_step": ms * 1e3, "tok_per_s": w.B / (ms * 1e-3), "host_read_bytes": host_read,
            "host_read_GBps": gbps, "frac_of_measured_read_peak": gbps / peak_read if peak_read else None,
            "frac_of_pcie5_x16": gbps / PCIE5_X16_GBPS,
            "overlap_model": _overlap_model(1, past, host_read, flops, MFMA_PEAK_TFLOPS[w.dtype], ms, peak_read)}


ATTN_SRC = ("attn.hip", "dkv_internal.h")
DECODE_SRC = ("decode.hip", "dkv_internal.h")


def _phase(t, name, steps):
    ms, n = t[name]
    if not n:
        return None
    return {"ms_per_step": ms / steps, "launches_per_step": n / steps, "avg_launch_ms": ms / n}


def _prefill_roofline(w, past, kern, name):
    """Prefill attention against the dtype's dense matrix-core peak: algorithmic attention flops
    per launch (the step's 4*d*Hq*sum_b(T*L_b + T(T+1)/2), spread over its launches) over the
    launches' mean duration (HIP events on the library's stream)."""
    from zero_copy_host_amd import accounting as acc
    a = kern.get("prefill_attention") if kern else None
    if not a:
        return None
    flops = acc.attention_flops(past, w.T, w.Hq, w.d)
    per_launch = flops / a["launches_per_step"]
    achieved = per_launch / (a["avg_launch_ms"] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    ctr = read_counter_summary(name, src_hash(*ATTN_SRC))
    return {"bound": "mfma", "kernel": "attn_kernel (prefill attention; every launch of a step)",
            "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
            "algorithmic_flops_per_launch": per_launch, "launches_per_step": a["launches_per_step"],
            "avg_launch_ms": a["avg_launch_ms"], "traffic": _float(ctr, "attn_fetch_plus_write_bytes_per_launch"),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
            "host_read_bytes_per_step_measured": _float(ctr, "host_read_bytes_per_step")}


def _decode_roofline(w, past, kern, peak_read, name):
    """The decode attention kernel against the host link: algorithmic host bytes per launch (every
    past K and V row once, 2*Hkv*d*e*sum_b L_b) over its mean duration (HIP events)."""
    import synth
    from zero_copy_host_amd import accounting as acc
    a = kern.get("decode_attention") if kern else None
    if not a:
        return None
    e = synth.elem_bytes(w.dtype)
    read = acc.host_read_bytes(past, w.Hkv, w.d, e)
    achieved = read / (a["avg_launch_ms"] * 1e-3) / 1e9
    ctr = read_counter_summary(name, src_hash(*DECODE_SRC))
    return {"bound": "host_link", "kernel": "decode_kernel", "achieved": achieved, "peak": PCIE5_X16_GBPS,
            "unit": "GB/s", "frac": achieved / PCIE5_X16_GBPS,
            "peak_note": "PCIe 5.0 x16 per direction; the measured kernel read peak is beside it",
            "measured_read_peak": peak_read, "frac_of_measured_read_peak": achieved / peak_read if peak_read else None,
            "algorithmic_bytes_per_launch": read + acc.host_write_bytes(w.B, 1, w.Hkv, w.d, e),
            "avg_launch_ms": a["avg_launch_ms"], "traffic": _float(ctr, "fetch_plus_write_bytes_per_launch"),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
            "host_read_bytes_measured": _float(ctr, "host_read_bytes_per_launch")}


def run_prefill(dkv, name, steps=5, warmup=2, peak_read=None, decode_steps=0, variant="fused",
                ablations=()):
    """Time the prefill step of workload `name` (fixed past lengths, so every step rewrites the
    same rows), with the library's kernel timing on; optionally follow it with real decode steps
    at advancing lengths."""
    import torch
    import synth
    w = synth.workload(name)
    past, cache, dev, dr = _layer_setup(dkv, w)
    out = torch.empty((w.B, w.T, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.workspace_bytes("prefill_staged" if variant == "staged" else "prefill", cache, w.B, w.T, w.Hq),
                     dtype=torch.uint8, device="cuda")

    def timed(var, n, nwarm, kernels=False):
        step = lambda: dkv.attn_prefill_variant(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out,
                                                ws, var)
        for _ in range(nwarm):
            step()
        torch.cuda.synchronize()
        with EventTimer() as t:
            for _ in range(n):
                step()
        # the kernel times come from a second pass of the same steps with the library's timing
        # events on (their recording costs host time, which would count in a launch-bound step)
        kern = {ph: _phase(tr, ph, n) for ph in ("projection", "prefill_attention")} if kernels and (
            tr := _timed_phases(dkv, step, n)) is not None else None
        return t.ms / n, kern

    ms, kern = timed(variant, steps, warmup, kernels=True)
    res = {"workload": name, "steps": steps, "variant": variant, **_prefill_stats(w, past, ms, peak_read),
           "kernels": kern, "roofline": _prefill_roofline(w, past, kern, name) if variant == "fused" else None}
    if ablations:
        # the baselines the pages compare the method against, on the same inputs
        res["ablations_ms"] = {}
        res["device_workspace_bytes"] = {variant: ws.numel()}
        for v in ablations:
            if v == "staged":   # needs a device copy of the whole cache in its workspace
                del ws
                torch.cuda.empty_cache()
                ws = torch.empty(dkv.workspace_bytes("prefill_staged", cache, w.B, w.T, w.Hq), dtype=torch.uint8,
                                 device="cuda")
                res["device_workspace_bytes"][v] = ws.numel()
            res["ablations_ms"][v] = timed(v, 2, 1)[0]
    if decode_steps:
        del out, ws
        xs = [to_dev(dr.normal((w.B, 1, w.D), 1.0, w.dtype), w.dtype) for _ in range(decode_steps)]
        outd = torch.empty((w.B, 1, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
        wsd = torch.empty(dkv.workspace_bytes("decode", cache, w.B, 1, w.Hq), dtype=torch.uint8, device="cuda")
        # one untimed call first (it writes the same row the first timed step rewrites)
        dkv.attn_decode(cache, xs[0], dev["wq"], dev["wk"], dev["wv"], past + w.T, w.Hq, outd, wsd)
        torch.cuda.synchronize()
        # a single decode step is timed as the mean of 20 runs of that step (same lengths, so
        # each run rewrites the same row); longer runs advance the lengths step by step
        reps = 20 if decode_steps == 1 else 1

        def steps_once():
            for _ in range(reps):
                for s_ in range(decode_steps):
                    dkv.attn_decode(cache, xs[s_], dev["wq"], dev["wk"], dev["wv"], past + w.T + s_, w.Hq, outd, wsd)
        with EventTimer() as t:
            steps_once()
        tr = _timed_phases(dkv, steps_once, 1)
        n = decode_steps * reps
        ms = t.ms / n
        mid = past + w.T + decode_steps // 2
        kd = {ph: _phase(tr, ph, n) for ph in ("decode_qproj", "decode_attention", "decode_combine")}
        res["decode"] = {"steps": decode_steps, "timed_runs": n, "past_len_first": int(past[0] + w.T),
                         **_decode_stats(w, mid, ms, peak_read), "kernels": kd,
                         "roofline": _decode_roofline(w, mid, kd, peak_read, name + "_decode")}
    cache.free()
    return res


def run_decode(dkv, name, steps=10, warmup=2, peak_read=None):
    """Time a decode step of workload `name` at fixed past lengths (every step rewrites the same
    new row), with the library's kernel timing on."""
    import torch
    import synth
    w = synth.workload(name)
    past, cache, dev, _ = _layer_setup(dkv, w)
    out = torch.empty((w.B, 1, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.workspace_bytes("decode", cache, w.B, 1, w.Hq), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        dkv.attn_decode(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    torch.cuda.synchronize()
    step = lambda: dkv.attn_decode(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    with EventTimer() as t:
        for _ in range(steps):
            step()
    tr = _timed_phases(dkv, step, steps)
    cache.free()
    kd = {ph: _phase(tr, ph, steps) for ph in ("decode_qproj", "decode_attention", "decode_combine")}
    return {"workload": name, "steps": steps, "past_len": [int(x) for x in past],
            **_decode_stats(w, past, t.ms / steps, peak_read), "kernels": kd,
            "roofline": _decode_roofline(w, past, kd, peak_read, name)}


def _paged_copy(dkv, w, past, cache, seed):
    """A page pool holding the rows of a filled contiguous cache through a shuffled block table
    (each sequence gets the pages this step needs, in random physical order)."""
    need = [(int(L) + w.T + dkv.PAGE_TOKENS - 1) // dkv.PAGE_TOKENS for L in past]
    total = sum(need)
    pool = dkv.PagedHostKVCache(total, w.Hkv, w.d, w.dtype)
    perm = np.random.default_rng(seed).permutation(total)
    lists, off = [], 0
    for n in need:
        lists.append(perm[off:off + n].tolist())
        off += n
    table = dkv.block_table(lists, max(need))
    for b, n in enumerate(need):
        rows = n * dkv.PAGE_TOKENS
        for src, dst in ((cache.k, pool.k), (cache.v, pool.v)):
            dst[table[b, :n]] = src[b, :, :rows].reshape(w.Hkv, n, dkv.PAGE_TOKENS, w.d).transpose(1, 0, 2, 3)
    return pool, table


def run_paged(dkv, peak_read=None, decode_steps=10, prefill_steps=3):
    """The 8B decode step and the 8B chunked prefill on a paged host cache (16-token pages in
    shuffled physical order), beside the contiguous numbers."""
    import torch
    import synth
    res = {}
    w = synth.workload("llama8b_decode_b8_L32768_bf16")
    past, cache, dev, _ = _layer_setup(dkv, w)
    pool, table = _paged_copy(dkv, w, past, cache, w.seed)
    cache.free()
    out = torch.empty((w.B, 1, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.paged_workspace_bytes("decode", pool, w.B, 1, w.Hq, table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    for _ in range(2):
        dkv.attn_decode_paged(pool, table, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    torch.cuda.synchronize()
    with EventTimer() as t:
        for _ in range(decode_steps):
            dkv.attn_decode_paged(pool, table, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    res["decode"] = {"workload": w.name, "steps": decode_steps, "pages": pool.n_pages,
                     **_decode_stats(w, past, t.ms / decode_steps, peak_read)}
    pool.free()
    del out, ws

    w = synth.workload("llama8b_prefill_T8192_on_L24576_bf16")
    past, cache, dev, _ = _layer_setup(dkv, w)
    pool, table = _paged_copy(dkv, w, past, cache, w.seed)
    cache.free()
    out = torch.empty((w.B, w.T, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.paged_workspace_bytes("prefill", pool, w.B, w.T, w.Hq, table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    dkv.attn_prefill_paged(pool, table, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    torch.cuda.synchronize()
    with EventTimer() as t:
        for _ in range(prefill_steps):
            dkv.attn_prefill_paged(pool, table, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    res["prefill"] = {"workload": w.name, "steps": prefill_steps, "pages": pool.n_pages,
                      **_prefill_stats(w, past, t.ms / prefill_steps, peak_read)}
    pool.free()
    return res


def run_staging(dkv, peak_read=None, steps=6):
    """The 8B decode step read zero-copy (this library) and through the staging baseline (the
    past rows DMA-copied into a device copy of the cache first, the new rows copied back): time
    per step and the device memory each call needs."""
    import torch
    import synth
    w = synth.workload("llama8b_decode_b8_L32768_bf16")
    past, cache, dev, _ = _layer_setup(dkv, w)
    out = torch.empty((w.B, 1, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    res = {"workload": w.name}
    for var, phase in (("zerocopy", "decode"), ("staged", "decode_staged")):
        nb = dkv.workspace_bytes(phase, cache, w.B, 1, w.Hq)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            dkv.attn_decode_variant(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws, var)
        torch.cuda.synchronize()
        with EventTimer() as t:
            for _ in range(steps):
                dkv.attn_decode_variant(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws, var)
        ms = t.ms / steps
        res[var] = {"us_per_step": ms * 1e3, "device_workspace_bytes": nb,
                    "host_bytes_per_step_GBps": _decode_stats(w, past, ms, peak_read)["host_read_GBps"]}
        del ws
        torch.cuda.empty_cache()
    res["staging_device_bytes"] = res["staged"]["device_workspace_bytes"] - res["zerocopy"]["device_workspace_bytes"]
    res["host_cache_bytes"] = cache.nbytes()
    cache.free()
    return res


STACKS = {
    # name: (layers, batch, past tokens, D, Hq, Hkv, d, F) -- Llama-3-8B- and 70B-shaped decoder stacks
    "llama8b_32layers_b8_L32768": (32, 8, 32768, 4096, 32, 8, 128, 14336),
    "llama70b_80layers_b2_L65536": (80, 2, 65536, 8192, 64, 8, 128, 28672),
}


def run_stack(dkv, name, tokens=3, peak_read=None):
    """Per-token latency of a full decoder stack in the decode phase: every layer has its own
    host KV cache (past K/V of layer 0 drawn from the workload seed and copied to the other
    layers; weights drawn on the device from a fixed seed, distinct per layer), and each token
    runs DecodeStack.step over all layers at advancing lengths."""
    import torch
    import synth
    from zero_copy_host_amd.decode_stack import DecodeStack
    n_layers, B, L, D, Hq, Hkv, d, F = STACKS[name]
    dt = "bf16"
    cap = (L + tokens + 63) // 64 * 64
    dr = synth.Draw(2000)
    caches = [dkv.HostKVCache(B, Hkv, d, cap, dt) for _ in range(n_layers)]
    past = np.full(B, L, dtype=np.int32)
    synth.fill_past(dr, caches[0].k, caches[0].v, past, dt)
    for c in caches[1:]:
        np.copyto(c.k, caches[0].k)
        np.copyto(c.v, caches[0].v)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2001)

    def w(out_f, in_f):
        return (torch.randn(out_f, in_f, generator=gen, device="cuda") * in_f ** -0.5).to(torch.bfloat16)

    layers = [{"wq": w(Hq * d, D), "wk": w(Hkv * d, D), "wv": w(Hkv * d, D), "wo": w(D, Hq * d),
               "w_gu": w(2 * F, D), "w_down": w(D, F),
               "g_attn": torch.ones(D, dtype=torch.bfloat16, device="cuda"),
               "g_mlp": torch.ones(D, dtype=torch.bfloat16, device="cuda")} for _ in range(n_layers)]
    weight_bytes = sum(t.numel() * t.element_size() for lw in layers for t in lw.values())
    stack = DecodeStack(layers, caches, Hq)
    h = torch.randn(B, D, generator=gen, device="cuda").to(torch.bfloat16)
    stack.step(h, past)                   # warm-up token at the first length (rewritten below)
    torch.cuda.synchronize()
    with EventTimer() as t:
        for i in range(tokens):
            stack.step(h, past + i)
    ms = t.ms / tokens
    host_read = n_layers * 2 * B * Hkv * (L + tokens // 2) * d * 2
    res = {"stack": name, "layers": n_layers, "batch": B, "past_len_first": L, "tokens": tokens,
           "ms_per_token": ms, "tok_per_s": B / (ms * 1e-3),
           "host_kv_bytes": sum(c.nbytes() for c in caches), "device_weight_bytes": weight_bytes,
           "host_read_GBps": host_read / (ms * 1e-3) / 1e9,
           "attention_share_note": "per layer: attn_decode (host-link bound) + norm/Wo/MLP (HBM)"}
    if peak_read:
        res["frac_of_measured_read_peak"] = res["host_read_GBps"] / peak_read
    del stack, layers, h
    for c in caches:
        c.free()
    torch.cuda.empty_cache()
    return res


def calibration_kernels(dkv, nbytes=1 << 30):
    """Kernels of known traffic for scaling the memory counters: one streaming read and one
    streaming write of nbytes of pinned host memory, and one device-to-device copy of
    nbytes (nbytes read + nbytes written in HBM)."""
    import torch
    buf = dkv.HostKVCache(1, 1, 128, nbytes // 256, "bf16")
    dkv.hostlink_stream(buf.desc.k, nbytes, "read", 1024)
    dkv.hostlink_stream(buf.desc.k, nbytes, "write", 1024)
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    buf.free()
    print(json.dumps({"calibration_bytes": nbytes}), flush=True)


def counters_summary(paths):
    """Per-kernel mean of every counter per dispatch over rocprofv3 --pmc CSV files, printed as
    JSON (the figures the counter summaries under profiles/ quote)."""
    import collections
    import csv
    out = {}
    for path in paths:
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        disp = collections.defaultdict(set)
        for r in csv.DictReader(open(path)):
            k = r["Kernel_Name"].split("(")[0]
            agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
        for k, cs in agg.items():
            n = len(disp[k])
            out.setdefault(k, {"dispatches": 0})
            out[k]["dispatches"] = max(out[k]["dispatches"], n)
            out[k].update({c: v / n for c, v in cs.items()})
    print(json.dumps(out, indent=1), flush=True)


HEADLINE = "llama70b_prefill_T16384_on_L49152_b2_bf16"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed prefill steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="the headline workload only")
    ap.add_argument("--variant", default="fused", choices=["fused", "naive", "separate", "staged"],
                    help="prefill variant for --profile prefill (the ablation baselines)")
    ap.add_argument("--profile", nargs="?", const="prefill",
                    choices=["decode", "prefill", "paged", "staging", "stack", "calib"],
                    help="short run for rocprofv3: prefill steps of --workload (default the headline), decode "
                         "steps of --workload (a decode workload), the paged-cache decode and prefill, the "
                         "staging baseline, the 8B/70B decoder stacks, or the counter calibration kernels "
                         "(1 GiB host read, 1 GiB host write, 1 GiB device-to-device copy)")
    ap.add_argument("--counters-summary", nargs="+", metavar="CSV",
                    help="print per-kernel per-dispatch means of rocprofv3 --pmc CSV files and exit")
    args = ap.parse_args()
    if args.counters_summary:
        counters_summary(args.counters_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the host-KV layer path runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import zero_copy_host_amd as dkv
    torch.cuda.set_device(0)
    dkv.lib()

    if args.profile == "calib":
        calibration_kernels(dkv)
        return
    if args.profile == "stack":
        out = {}
        for name in STACKS:
            log(f"decoder stack {name}")
            out[name] = run_stack(dkv, name, tokens=max(1, args.steps))
        print(json.dumps({"decode_stack": out}), flush=True)
        return
    if args.profile == "staging":
        print(json.dumps({"staging_baseline": run_staging(dkv, steps=args.steps),
                          "prefill": run_prefill(dkv, "llama8b_prefill_T8192_on_L24576_bf16", steps=3, warmup=1,
                                                 ablations=("staged",))}), flush=True)
        return
    if args.profile == "paged":
        print(json.dumps({"paged": run_paged(dkv, decode_steps=args.steps, prefill_steps=max(1, args.steps // 3))}),
              flush=True)
        return
    if args.profile == "prefill":
        name = args.workload if synth.workload(args.workload).T > 1 else HEADLINE
        print(json.dumps({"prefill": run_prefill(dkv, name, steps=args.steps,
                                                 warmup=args.warmup, variant=args.variant)}), flush=True)
        return
    if args.profile == "decode":
        name = args.workload if synth.workload(args.workload).T == 1 else "llama8b_decode_b8_L32768_bf16"
        print(json.dumps({"decode": run_decode(dkv, name, steps=args.steps, warmup=args.warmup)}), flush=True)
        return

    log("measuring host-link peak")
    peak = hostlink_peak(dkv)
    pr = peak["read"]
    w = synth.workload(args.workload)
    assert w.T > 1, "the headline workload is a prefill step"
    log(f"{w.name}: {args.warmup} warmup and {args.steps} timed prefill steps, then {w.decode_steps} decode steps")
    head = run_prefill(dkv, w.name, steps=args.steps, warmup=args.warmup, peak_read=pr, decode_steps=w.decode_steps)
    ms = head["ms_per_step"]
    result = {
        "metric": "prefill tok/s & decode step us per layer; host-link GB/s vs measured peak",
        "value": head["tok_per_s"],
        "unit": "prefill tok/s per layer (B*T new tokens / step time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) X and past K/V, N(0,1/D) weights)",
        "config": {"workload": w.name, "batch": w.B, "new_tokens": w.T, "past_len": int(w.past[0]),
                   "decode_steps_after": w.decode_steps, "D": w.D, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.d,
                   "kv_cache": "pinned host memory"},
        "roofline": head["roofline"],
        "prefill": {k: v for k, v in head.items() if k not in ("roofline", "decode")},
        "decode": head.get("decode"),
        "host_link": {"kernel_read_GBps": peak["read"], "kernel_write_GBps": peak["write"]},
    }
    if not args.no_others:
        others = {}
        log("8B-shaped decode, B=8, L=32768")
        others["llama8b_decode_b8_L32768_bf16"] = run_decode(dkv, "llama8b_decode_b8_L32768_bf16", steps=20,
                                                              warmup=3, peak_read=pr)
        log("8B-shaped chunked prefill and its ablations")
        others["llama8b_prefill_T8192_on_L24576_bf16"] = run_prefill(
            dkv, "llama8b_prefill_T8192_on_L24576_bf16", steps=5, warmup=2, peak_read=pr,
            ablations=("naive", "separate", "staged"))
        log("long-context fp16 decode")
        others["long_decode_b4_L96k_128k_f16"] = run_decode(dkv, "long_decode_b4_L96k_128k_f16", steps=6, warmup=1,
                                                             peak_read=pr)
        log("tiny fp32 layer")
        others["tiny_f32_prefill128_decode1"] = run_prefill(dkv, "tiny_f32_prefill128_decode1", steps=20, warmup=3,
                                                            peak_read=pr, decode_steps=1)
        log("70B-shaped prefill from an empty cache + 64 decode steps (the other reading of that case)")
        others["llama70b_prefill_T16384_empty_b2_bf16"] = run_prefill(
            dkv, "llama70b_prefill_T16384_empty_b2_bf16", steps=2, warmup=1, peak_read=pr, decode_steps=64)
        log("paged host cache: 8B decode and 8B chunked prefill")
        result["paged"] = run_paged(dkv, peak_read=pr)
        log("staging baseline: 8B decode")
        result["staging_baseline"] = run_staging(dkv, peak_read=pr)
        log("decoder stack: 32 layers of the 8B layer, per-token latency")
        result["decode_stack"] = {"llama8b_32layers_b8_L32768": run_stack(dkv, "llama8b_32layers_b8_L32768",
                                                                          tokens=2, peak_read=pr)}
        result["workloads"] = others
    if not args.no_cpu_baseline:
        # after every GPU measurement: the oracle's threads on the host cores would otherwise slow
        # the kernel launches of the launch-bound workloads
        log("timing the oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline_prefill(w.name)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
