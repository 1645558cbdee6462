"""Benchmark of the host-KV attention layer on one MI355X.

Default workload: a Llama-3-8B-shaped layer decode step in bf16 (D=4096, Hq=32, Hkv=8,
d=128), batch 8, 32768 past tokens per sequence held in pinned host memory. A step is one
attn_decode call: q/k/v projection of the new token, append of k/v to the host cache,
split-KV attention over all 32769 keys, and the combine. Inputs are synthetic (seeded
N(0,1) activations and past K/V, N(0, 1/D) weights) and resident before timing starts:
X and W in device memory, the KV cache in pinned host memory, where the method keeps it.

Prints one JSON line. Extra objects: the measured host-link peak (kernel streaming
read/write of pinned memory), the roofline of the decode kernel, the oracle timed on the
host cores (cpu_baseline), and a chunked-prefill measurement (8192 new tokens on 24576
host-resident past tokens) for the prefill half of the metric.
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
PROFILE_NOTE = os.path.join(ROOT, "profiles", "decode_llama8b_b8_L32768_counters.txt")


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


def setup_decode(dkv, w, seed_off=0):
    import synth
    dr = synth.Draw(w.seed + seed_off)
    wq, wk, wv = synth.layer_weights(dr, w.D, w.Hq, w.Hkv, w.d, w.dtype)
    past = np.asarray(w.past, dtype=np.int32) if w.past is not None else dr.lengths(w.B, w.past_lo, w.past_hi)
    x = dr.normal((w.B, 1, w.D), 1.0, w.dtype)
    cache = dkv.HostKVCache(w.B, w.Hkv, w.d, w.cap, w.dtype)
    synth.fill_past(dr, cache.k, cache.v, past, w.dtype)
    return dict(wq=wq, wk=wk, wv=wv, x=x, past=past, cache=cache)


def cpu_baseline_decode(w, s, min_seconds=10.0):
    """The oracle, as it is, on the same decode step, repeated for ~min_seconds."""
    import oracle
    import synth
    import threadpoolctl
    kc = synth.from_storage(s["cache"].k, w.dtype)
    vc = synth.from_storage(s["cache"].v, w.dtype)
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.layer_step(s["x"], s["wq"], s["wk"], s["wv"], kc, vc, s["past"], w.Hq, w.dtype)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {"value": el / n * 1e6, "unit": "us/layer-step", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full decode step(s) of the same workload (all {w.B} sequences, "
                      f"{int(s['past'][0]) + 1} keys each) in fp64 numpy; host has {os.cpu_count()} cpus"}


def profile_traffic(kernel_src_hash):
    """HBM/host bytes per decode launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(PROFILE_NOTE):
        return None, None
    vals = {}
    for line in open(PROFILE_NOTE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha1") != kernel_src_hash:
        return None, None
    try:
        return float(vals["fetch_plus_write_bytes_per_launch"]), float(vals["host_read_bytes_per_launch"])
    except (KeyError, ValueError):
        return None, None


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


def run_prefill(dkv, name, steps=5, warmup=2, peak_read=None, decode_steps=0, variant="fused",
                ablations=()):
    """Time the prefill step of workload `name` (fixed past lengths, so every step rewrites the
    same rows); optionally follow it with real decode steps at advancing lengths."""
    import torch
    import synth
    w = synth.workload(name)
    past, cache, dev, dr = _layer_setup(dkv, w)
    out = torch.empty((w.B, w.T, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.workspace_bytes("prefill_staged" if variant == "staged" else "prefill", cache, w.B, w.T, w.Hq),
                     dtype=torch.uint8, device="cuda")
    def timed(var, n, nwarm):
        for _ in range(nwarm):
            dkv.attn_prefill_variant(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws, var)
        torch.cuda.synchronize()
        with EventTimer() as t:
            for _ in range(n):
                dkv.attn_prefill_variant(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws, var)
        return t.ms / n

    res = {"workload": name, "steps": steps, "variant": variant,
           **_prefill_stats(w, past, timed(variant, steps, warmup), peak_read)}
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
            res["ablations_ms"][v] = timed(v, 2, 1)
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
        with EventTimer() as t:
            for _ in range(reps):
                for s_ in range(decode_steps):
                    dkv.attn_decode(cache, xs[s_], dev["wq"], dev["wk"], dev["wv"], past + w.T + s_, w.Hq, outd, wsd)
        ms = t.ms / (decode_steps * reps)
        mid = past + w.T + decode_steps // 2
        res["decode"] = {"steps": decode_steps, "timed_runs": decode_steps * reps, "past_len_first": int(past[0] + w.T),
                         **_decode_stats(w, mid, ms, peak_read)}
    cache.free()
    return res


def run_decode(dkv, name, steps=10, warmup=2, peak_read=None):
    """Time a decode step of workload `name` at fixed past lengths."""
    import torch
    import synth
    w = synth.workload(name)
    past, cache, dev, _ = _layer_setup(dkv, w)
    out = torch.empty((w.B, 1, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.workspace_bytes("decode", cache, w.B, 1, w.Hq), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        dkv.attn_decode(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    torch.cuda.synchronize()
    with EventTimer() as t:
        for _ in range(steps):
            dkv.attn_decode(cache, dev["x"], dev["wq"], dev["wk"], dev["wv"], past, w.Hq, out, ws)
    cache.free()
    return {"workload": name, "steps": steps, "past_len": [int(x) for x in past],
            **_decode_stats(w, past, t.ms / steps, peak_read)}


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


def bench_prefill(dkv, steps=5, warmup=2):
    return run_prefill(dkv, "llama8b_prefill_T8192_on_L24576_bf16", steps, warmup)


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_decode_b8_L32768_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", default="fused", choices=["fused", "naive", "separate", "staged"],
                    help="prefill variant for --profile prefill (the ablation baselines)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--profile", nargs="?", const="decode", choices=["decode", "prefill", "paged", "staging", "stack", "calib"],
                    help="short run for rocprofv3: decode steps only, prefill steps only, the paged-cache "
                         "decode and prefill, the staging baseline, the 8B/70B decoder stacks, or the "
                         "counter calibration kernels (1 GiB host read, 1 GiB host write, 1 GiB "
                         "device-to-device copy)")
    args = ap.parse_args()
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
        # the 8B chunked prefill unless --workload names another prefill workload
        name = args.workload if synth.workload(args.workload).T > 1 else "llama8b_prefill_T8192_on_L24576_bf16"
        print(json.dumps({"prefill": run_prefill(dkv, name, steps=args.steps,
                                                 warmup=args.warmup, variant=args.variant)}), flush=True)
        return
    if args.profile:
        args.no_cpu_baseline = args.no_prefill = True

    peak = {"read": None, "write": None}
    if not args.profile:
        log("measuring host-link peak")
        peak = hostlink_peak(dkv)

    w = synth.workload(args.workload)
    assert w.T == 1, "the timed workload is a decode step"
    log(f"setting up {w.name}")
    s = setup_decode(dkv, w)
    xd = to_dev(s["x"], w.dtype)
    wqd, wkd, wvd = to_dev(s["wq"].T, w.dtype), to_dev(s["wk"].T, w.dtype), to_dev(s["wv"].T, w.dtype)
    out = torch.empty((w.B, 1, w.Hq * w.d), dtype=tdtype(w.dtype), device="cuda")
    ws = torch.empty(dkv.workspace_bytes("decode", s["cache"], w.B, 1, w.Hq), dtype=torch.uint8, device="cuda")
    past = s["past"]

    def step():
        # fixed lengths: every step rewrites the same new-token row
        dkv.attn_decode(s["cache"], xd, wqd, wkd, wvd, past, w.Hq, out, ws)

    log(f"warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    with EventTimer() as t:
        for _ in range(args.steps):
            step()
    ms = t.ms / args.steps
    torch.cuda.synchronize()

    from zero_copy_host_amd import accounting as acc
    e = synth.elem_bytes(w.dtype)
    host_read = acc.host_read_bytes(past, w.Hkv, w.d, e)         # every past row, K and V, once
    host_write = acc.host_write_bytes(w.B, 1, w.Hkv, w.d, e)     # the new row
    achieved = host_read / (ms * 1e-3) / 1e9
    traffic, host_meas = profile_traffic(src_hash("decode.hip", "dkv_internal.h"))
    result = {
        "metric": "prefill tok/s & decode step us per layer; host-link GB/s vs measured peak",
        "value": ms * 1e3,
        "unit": "us per layer decode step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) X and past K/V, N(0,1/D) weights)",
        "config": {"workload": w.name, "batch": w.B, "past_len": int(past[0]), "new_tokens": 1,
                   "D": w.D, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.d, "kv_cache": "pinned host memory"},
        "decode_tok_per_s": w.B / (ms * 1e-3),
        "overlap_model": _overlap_model(
            1, past, host_read, acc.attention_flops(past, 1, w.Hq, w.d) + acc.projection_flops(w.B, 1, w.D, w.Hq, w.Hkv, w.d),
            MFMA_PEAK_TFLOPS[w.dtype], ms, peak["read"]),
        "roofline": {"bound": "host_link", "kernel": "decode_kernel (+ qproj_kernel, combine_kernel) per attn_decode call",
                     "achieved": achieved, "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                     "frac": achieved / PCIE5_X16_GBPS,
                     "peak_note": "PCIe 5.0 x16 per direction; measured kernel read peak below",
                     "measured_read_peak": peak["read"],
                     "frac_of_measured_read_peak": (achieved / peak["read"]) if peak["read"] else None,
                     "algorithmic_bytes_per_launch": host_read + host_write,
                     "traffic": traffic, "host_read_bytes_measured": host_meas},
        "host_link": {"kernel_read_GBps": peak["read"], "kernel_write_GBps": peak["write"]},
    }
    if not args.no_prefill:
        pr = peak["read"]
        log("other workloads: tiny fp32 layer")
        tiny = run_prefill(dkv, "tiny_f32_prefill128_decode1", steps=20, warmup=3, peak_read=pr, decode_steps=1)
        log("8B chunked prefill")
        result["prefill"] = run_prefill(dkv, "llama8b_prefill_T8192_on_L24576_bf16", steps=5, warmup=2, peak_read=pr,
                                        ablations=("naive", "separate", "staged"))
        log("staging baseline: 8B decode")
        result["staging_baseline"] = run_staging(dkv, peak_read=pr)
        log("decoder stack: 32 layers of the 8B layer, per-token latency")
        result["decode_stack"] = {"llama8b_32layers_b8_L32768": run_stack(dkv, "llama8b_32layers_b8_L32768",
                                                                          tokens=2, peak_read=pr)}
        log("long-context fp16 decode")
        longd = run_decode(dkv, "long_decode_b4_L96k_128k_f16", steps=6, warmup=1, peak_read=pr)
        log("70B prefill + 64 decode steps")
        big = run_prefill(dkv, "llama70b_prefill_T16384_on_L49152_b2_bf16", steps=2, warmup=1, peak_read=pr,
                          decode_steps=64)
        log("70B prefill from an empty cache + 64 decode steps (the other reading of that case)")
        big0 = run_prefill(dkv, "llama70b_prefill_T16384_empty_b2_bf16", steps=2, warmup=1, peak_read=pr,
                           decode_steps=64)
        log("paged host cache: 8B decode and 8B chunked prefill")
        result["paged"] = run_paged(dkv, peak_read=pr)
        result["workloads"] = {"tiny_f32_prefill128_decode1": tiny,
                               "llama8b_prefill_T8192_on_L24576_bf16": result["prefill"],
                               "long_decode_b4_L96k_128k_f16": longd,
                               "llama70b_prefill_T16384_on_L49152_b2_bf16": big,
                               "llama70b_prefill_T16384_empty_b2_bf16": big0}
    if not args.no_cpu_baseline:
        # after every GPU measurement: the oracle's threads on all host cores would otherwise
        # slow the kernel launches of the launch-bound workloads measured after it
        log("timing the oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline_decode(w, s)
    s["cache"].free()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
