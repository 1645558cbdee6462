"""The staging baseline (past KV copied into device memory before the kernels run, new rows
copied back) against the zero-copy path, through the C ABI: the same kernels on the same
values, so outputs and host cache rows must be bit-identical; the only difference is the
device memory the staging copy takes.
"""
import numpy as np
import pytest

import synth
from gpu_case import GpuLayer, compare, oracle_step, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype):
    cap = ((max(past) + T + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap)


def _run(case, phase, variant):
    import torch
    g = GpuLayer(case)
    try:
        c = case
        B, T = c["B"], c["T"]
        xd = to_dev(c["x"], c["dtype"])
        out = torch.empty((B, T, c["Hq"] * c["d"]), dtype=torch_dtype(c["dtype"]), device="cuda")
        staged = variant == "staged"
        nb = g.dkv.workspace_bytes(phase + ("_staged" if staged else ""), g.cache, B, T, c["Hq"])
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        if phase == "decode":
            g.dkv.attn_decode_variant(g.cache, xd, g.wq, g.wk, g.wv, c["past_len"], c["Hq"], out, ws,
                                      "staged" if staged else "zerocopy")
        else:
            g.dkv.attn_prefill_variant(g.cache, xd, g.wq, g.wk, g.wv, c["past_len"], c["Hq"], out, ws,
                                       "staged" if staged else "fused")
        torch.cuda.synchronize()
        return (out.float().cpu().numpy().reshape(B, T, c["Hq"], c["d"]), g.cache.k.copy(), g.cache.v.copy(), nb)
    finally:
        g.free()


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f32", 64, 2)])
def test_staged_decode_equals_zero_copy_bitwise(dtype, d, G):
    case = _case(401, 3, 1, [100, 37, 250], 256, 2 * G, 2, d, dtype)
    out_z, k_z, v_z, nb_z = _run(case, "decode", "zerocopy")
    out_s, k_s, v_s, nb_s = _run(case, "decode", "staged")
    assert np.array_equal(out_s, out_z)
    assert np.array_equal(k_s, k_z) and np.array_equal(v_s, v_z)   # the new rows landed on the host
    # the staging copy of the whole cache (K and V) is the extra device memory
    cache_bytes = 2 * case["B"] * case["Hkv"] * case["cap"] * d * synth.elem_bytes(dtype)
    assert nb_s - nb_z >= cache_bytes and nb_s - nb_z < cache_bytes + 1024
    kc, vc = case["kp"].copy(), case["vp"].copy()
    compare(out_s, oracle_step(case, case["x"], case["past_len"], kc, vc), dtype, f"staged decode {dtype}")


def test_staged_prefill_equals_fused_bitwise():
    case = _case(402, 2, 70, [33, 130], 256, 8, 2, 128, "bf16")
    out_f, k_f, v_f, _ = _run(case, "prefill", "fused")
    out_s, k_s, v_s, _ = _run(case, "prefill", "staged")
    assert np.array_equal(out_s, out_f)
    assert np.array_equal(k_s, k_f) and np.array_equal(v_s, v_f)
    kc, vc = case["kp"].copy(), case["vp"].copy()
    compare(out_s, oracle_step(case, case["x"], case["past_len"], kc, vc), "bf16", "staged prefill")
