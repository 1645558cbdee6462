"""The decode-loop kernels (RMSNorm, linear with residual, SwiGLU) and a two-layer decoder stack
(DecodeStack: one host KV cache per layer, with and without the rotary embedding) against the
oracle, through the C ABI.

Tolerances. Each kernel accumulates in fp32 and rounds once to the storage dtype, as the oracle
(fp64) does at the same points: a single kernel is within 1 ulp of the dtype plus the fp32
accumulation error (K·2⁻²⁴·Σ|x||w| for a K-term product). A decoder layer is checked on its own,
fed the GPU's own input to that layer, so errors do not compound across layers: its output
differs from the oracle's by the attention output's error carried through Wo (Wo ~ N(0, 1/(Hq·d))
keeps a random error's size: the layer's attention tolerance, max-abs 2e-2 / mean-abs 2e-3 for
bf16, 1e-5 for fp32) plus the two residual sums' roundings, each of which can land one ulp of
the hidden state away from the oracle's; the MLP's roundings feed the second sum the same way.
The whole stack is then the chain of its layers, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import _ulp, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    return to_dev(np.ascontiguousarray(a), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm_kernel(dtype):
    import zero_copy_host_amd as dkv
    dr = synth.Draw(501)
    x = dr.normal((5, 1000), 2.0, dtype)
    g = synth.quantize(1.0 + dr.normal((1000,), 0.1, "f32"), dtype)
    xd, gd = _dev(x, dtype), _dev(g, dtype)
    y = xd.clone()
    dkv.rmsnorm(xd, gd, y, 1e-5)
    got = from_dev(y)
    ref = oracle.rmsnorm(x, g, 1e-5)
    # one rounding of a value computed in fp32 (relative error a few 2^-24)
    assert (np.abs(got - ref) <= _ulp(ref, dtype) + 1e-6 * np.abs(ref)).all()
    dkv.rmsnorm(xd, gd, xd, 1e-5)          # in place
    assert np.array_equal(from_dev(xd), got)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows", [1, 3, 8, 13, 21])
def test_linear_kernel_with_residual(dtype, rows):
    import zero_copy_host_amd as dkv
    dr = synth.Draw(502 + rows)
    K, N = 384, 200
    x = dr.normal((rows, K), 1.0, dtype)
    w = dr.weights(K, N, dtype)                      # [in, out]
    r = dr.normal((rows, N), 1.0, dtype)
    xd, wd, rd = _dev(x, dtype), _dev(w.T, dtype), _dev(r, dtype)
    y = rd.clone()
    dkv.linear(xd, wd, y, residual=y)                # in-place residual add
    got = from_dev(y)
    exact = oracle.project(x, w) + r
    bound = K * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w)) + _ulp(exact, dtype)
    assert (np.abs(got - exact) <= bound).all()
    y2 = rd.clone()
    dkv.linear(xd, wd, y2)                           # no residual
    got2 = from_dev(y2)
    exact2 = oracle.project(x, w)
    assert (np.abs(got2 - exact2) <= K * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w)) + _ulp(exact2, dtype)).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swiglu_kernel(dtype):
    import torch
    import zero_copy_host_amd as dkv
    dr = synth.Draw(503)
    gu = dr.normal((4, 2 * 300), 3.0, dtype)
    gd = _dev(gu, dtype)
    y = torch.empty((4, 300), dtype=gd.dtype, device="cuda")
    dkv.swiglu(gd, y)
    got = from_dev(y)
    ref = oracle.swiglu(gu)
    assert (np.abs(got - ref) <= _ulp(ref, dtype) + 1e-6 * np.abs(ref) + 1e-30).all()


def test_helpers_reject_bad_arguments():
    import ctypes
    import torch
    import zero_copy_host_amd as dkv
    L = dkv.lib()
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    assert L.dkv_linear(a.data_ptr(), b.data_ptr(), None, a.data_ptr(), 4, 64, 64, 2, None) == -1   # y overlaps x
    assert L.dkv_linear(a.data_ptr(), b.data_ptr(), None, b.data_ptr(), 4, 64, 60, 2, None) == -1   # K*2 % 16
    assert L.dkv_linear(a.data_ptr(), b.data_ptr(), None, b.data_ptr(), 4, 64, 64, 9, None) == -3   # dtype
    assert L.dkv_swiglu(a.data_ptr(), a.data_ptr(), 4, 32, 2, None) == -1                           # overlap
    assert L.dkv_rmsnorm(None, b.data_ptr(), a.data_ptr(), 4, 64, ctypes.c_float(1e-5), 2, None) == -1


def _stack_case(dtype, n_layers=2, B=3, D=256, Hq=8, Hkv=2, d=64, F=384):
    past = np.array([37, 100, 5], dtype=np.int32)[:B]
    cap = 192
    dr = synth.Draw(504)
    layers = synth.stack_weights(dr, n_layers, D, Hq, Hkv, d, F, dtype)
    caches_o = []
    for _ in range(n_layers):
        kc = np.zeros((B, Hkv, cap, d), dtype=np.float32)
        vc = np.zeros((B, Hkv, cap, d), dtype=np.float32)
        synth.fill_past(dr, kc, vc, past, dtype)
        caches_o.append((kc, vc))
    h = dr.normal((B, D), 1.0, dtype)
    return dict(layers=layers, caches_o=caches_o, h=h, past=past, B=B, D=D, Hq=Hq, Hkv=Hkv, d=d, cap=cap)


def _host_caches(case, dtype):
    import zero_copy_host_amd as dkv
    out = []
    for kc, vc in case["caches_o"]:
        c = dkv.HostKVCache(case["B"], case["Hkv"], case["d"], case["cap"], dtype)
        c.k[...] = synth.to_storage(kc, dtype)
        c.v[...] = synth.to_storage(vc, dtype)
        out.append(c)
    return out


def _dev_layer(lw, dtype):
    return {"wq": _dev(lw["wq"].T, dtype), "wk": _dev(lw["wk"].T, dtype), "wv": _dev(lw["wv"].T, dtype),
            "wo": _dev(lw["wo"].T, dtype), "w_gu": _dev(lw["w_gu"].T, dtype),
            "w_down": _dev(lw["w_down"].T, dtype), "g_attn": _dev(lw["g_attn"], dtype),
            "g_mlp": _dev(lw["g_mlp"], dtype)}


@pytest.mark.parametrize("rope_theta", [0.0, 500000.0], ids=["norope", "rope"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_layer_decode_stack(dtype, rope_theta):
    import torch
    from zero_copy_host_amd.decode_stack import DecodeStack
    case = _stack_case(dtype)
    layers, past, Hq = case["layers"], case["past"], case["Hq"]
    dev_layers = [_dev_layer(lw, dtype) for lw in layers]
    tmax, tmean = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}[dtype]

    # each layer alone (a one-layer stack on fresh caches), fed the GPU's output of the layer before
    h_in = case["h"]
    chain = []
    for i, lw in enumerate(layers):
        caches = _host_caches(case, dtype)
        try:
            one = DecodeStack([dev_layers[i]], [caches[i]], Hq, eps=1e-5, rope_theta=rope_theta)
            hd = _dev(h_in, dtype)
            one.step(hd, past)
            torch.cuda.synchronize()
            h_out = from_dev(hd)
            kg, vg = synth.from_storage(caches[i].k, dtype), synth.from_storage(caches[i].v, dtype)
        finally:
            for c in caches:
                c.free()
        ko, vo = case["caches_o"][i][0].copy(), case["caches_o"][i][1].copy()
        ref = oracle.decode_stack_step(h_in, [lw], [(ko, vo)], past, Hq, dtype, 1e-5, rope_theta=rope_theta)
        err = np.abs(h_out - ref)
        ulp = _ulp(ref, dtype)
        print(f"layer {i} {dtype} rope={rope_theta}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
        assert (err <= tmax + 2 * ulp).all(), f"layer {i}: max-abs {err.max():.3e}"
        assert err.mean() <= tmean + float(ulp.mean()), f"layer {i}: mean-abs {err.mean():.3e}"
        # the layer appended the new token's K/V at row past_len[b] and touched nothing else; the
        # appended rows come from the normed input, computed in fp32 on both sides of one rounding
        for b, L in enumerate(past):
            assert np.array_equal(kg[b, :, :L], ko[b, :, :L]) and np.array_equal(vg[b, :, :L], vo[b, :, :L])
            assert np.all(kg[b, :, L + 1:] == 0) and np.all(vg[b, :, L + 1:] == 0)
            assert np.abs(kg[b, :, L] - ko[b, :, L]).max() <= tmax
            assert np.abs(vg[b, :, L] - vo[b, :, L]).max() <= tmax
        chain.append(h_out)
        h_in = h_out

    # the two-layer stack is the chain of its layers, bit for bit
    caches = _host_caches(case, dtype)
    try:
        stack = DecodeStack(dev_layers, caches, Hq, eps=1e-5, rope_theta=rope_theta)
        hd = _dev(case["h"], dtype)
        stack.step(hd, past)
        torch.cuda.synchronize()
        got = from_dev(hd)
    finally:
        for c in caches:
            c.free()
    assert np.array_equal(got, chain[-1])
