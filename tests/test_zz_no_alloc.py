"""attn_decode_noalloc (no workspace argument; the library's per-GPU device scratch holds the
partials) against attn_decode, through the C ABI: the same kernels on the same inputs, so the
outputs and the appended rows must be bitwise equal. Two calls in a row, the second smaller, so
the second runs over the first one's leftovers in the scratch; then a call beyond the scratch
size is refused before anything is enqueued."""
import numpy as np
import pytest

import synth
from gpu_case import GpuLayer, compare, oracle_step, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _decode_both(case):
    """(attn_decode output, attn_decode_noalloc output, cache rows after each) on one case."""
    import torch
    import zero_copy_host_amd as dkv
    c = case
    outs, rows = [], []
    for fn in ("ws", "noalloc"):
        g = GpuLayer(c)
        try:
            x = to_dev(c["x"], c["dtype"])
            out = torch.full((c["B"], 1, c["Hq"] * c["d"]), float("nan"), dtype=torch_dtype(c["dtype"]),
                             device="cuda")
            if fn == "ws":
                ws = torch.empty(dkv.workspace_bytes("decode", g.cache, c["B"], 1, c["Hq"]), dtype=torch.uint8,
                                 device="cuda")
                dkv.attn_decode(g.cache, x, g.wq, g.wk, g.wv, c["past_len"], c["Hq"], out, ws)
            else:
                dkv.attn_decode_noalloc(g.cache, x, g.wq, g.wk, g.wv, c["past_len"], c["Hq"], out)
            torch.cuda.synchronize()
            outs.append(out.view(torch.int16 if c["dtype"] != "f32" else torch.int32).cpu().numpy())
            rows.append((g.cache.k.copy(), g.cache.v.copy()))
            last = out.float().cpu().numpy().reshape(c["B"], 1, c["Hq"], c["d"])
        finally:
            g.free()
    return outs, rows, last


def _case(seed, B, past, D, Hq, Hkv, d, dtype):
    cap = ((max(past) + 1 + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, 1, past, D, Hq, Hkv, d, dtype, cap)


def test_noalloc_equals_workspace_call_twice_then_smaller():
    cases = [
        _case(41, 8, [3000, 9000, 5000, 7000, 4100, 8800, 6000, 3500], 512, 32, 8, 128, "bf16"),   # several splits
        _case(42, 2, [100, 2500], 256, 8, 2, 128, "f16"),                                           # smaller
        _case(43, 1, [40], 256, 4, 4, 64, "f32"),                                                   # one split
    ]
    for i, case in enumerate(cases):
        print(f"no-alloc decode call {i}: B={case['B']} past={case['past_len'].tolist()} {case['dtype']}", flush=True)
        outs, rows, got = _decode_both(case)
        assert np.array_equal(outs[0], outs[1]), f"call {i}: output differs from attn_decode"
        for b in range(case["B"]):
            L = int(case["past_len"][b])
            assert np.array_equal(rows[0][0][b, :, L], rows[1][0][b, :, L]), f"call {i}: appended K row"
            assert np.array_equal(rows[0][1][b, :, L], rows[1][1][b, :, L]), f"call {i}: appended V row"
        kc, vc = case["kp"].copy(), case["vp"].copy()
        compare(got, oracle_step(case, case["x"], case["past_len"], kc, vc), case["dtype"], f"no-alloc call {i}")


def test_noalloc_refuses_calls_beyond_its_scratch():
    import torch
    import zero_copy_host_amd as dkv
    B, Hkv, Hq, d, D = 256, 8, 64, 128, 256
    cache = dkv.HostKVCache(B, Hkv, d, 64, "bf16")
    try:
        bf = torch.bfloat16
        x = torch.zeros(B, 1, D, dtype=bf, device="cuda")
        wq = torch.zeros(Hq * d, D, dtype=bf, device="cuda")
        wk = torch.zeros(Hkv * d, D, dtype=bf, device="cuda")
        out = torch.zeros(B, 1, Hq * d, dtype=bf, device="cuda")
        with pytest.raises(dkv.DirectKVError) as ei:
            dkv.attn_decode_noalloc(cache, x, wq, wk, wk, np.full(B, 10, np.int32), Hq, out)
        assert ei.value.status == -6 and "scratch" in str(ei.value)
        torch.cuda.synchronize()
        assert not bool(out.abs().sum().item()), "a refused call enqueued work"
    finally:
        cache.free()
