"""Helpers for GPU parity tests: run a layer step through the C ABI (HIP path) and through
the oracle on the same seeded inputs, and compare.

Only input generation (synth) is shared by the two sides.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

# tolerances against the fp64 oracle: max-abs and mean-abs for 16-bit types, max-abs for fp32
TOL = {"bf16": (2e-2, 2e-3), "f16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}

NAN_BITS = {"bf16": np.uint16(0x7FC1), "f16": np.uint16(0x7E01)}


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(dtype)).cuda()


def from_dev(t):
    return t.float().cpu().numpy()


def fill_canary(arr, dtype):
    if dtype == "f32":
        arr[...] = np.float32(np.nan)
    else:
        arr[...] = NAN_BITS[dtype]


class GpuLayer:
    """A host cache plus device copies of X and the weights for one case."""

    def __init__(self, case, canary: bool = False):
        import zero_copy_host_amd as dkv
        self.dkv = dkv
        self.c = c = case
        dt = c["dtype"]
        self.cache = dkv.HostKVCache(c["B"], c["Hkv"], c["d"], c["cap"], dt)
        if canary:
            fill_canary(self.cache.k, dt)
            fill_canary(self.cache.v, dt)
        for b in range(c["B"]):
            L = int(c["past_len"][b])
            for g in range(c["Hkv"]):
                self.cache.k[b, g, :L] = synth.to_storage(c["kp"][b, g, :L], dt)
                self.cache.v[b, g, :L] = synth.to_storage(c["vp"][b, g, :L], dt)
        # weights go to the device in the [out, in] layout the ABI takes
        self.wq = to_dev(c["wq"].T, dt)
        self.wk = to_dev(c["wk"].T, dt)
        self.wv = to_dev(c["wv"].T, dt)

    def prefill(self, x, past_len, variant=None, rope_theta=0.0):
        import torch
        c = self.c
        B, T, D = x.shape
        xd = to_dev(x, c["dtype"])
        out = torch.empty((B, T, c["Hq"] * c["d"]), dtype=torch_dtype(c["dtype"]), device="cuda")
        nb = self.dkv.workspace_bytes("prefill", self.cache, B, T, c["Hq"])
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        if variant is None:
            self.dkv.attn_prefill(self.cache, xd, self.wq, self.wk, self.wv, past_len, c["Hq"], out, ws,
                                  rope_theta=rope_theta)
        else:
            self.dkv.attn_prefill_variant(self.cache, xd, self.wq, self.wk, self.wv, past_len, c["Hq"], out, ws,
                                          variant)
        torch.cuda.synchronize()
        return from_dev(out).reshape(B, T, c["Hq"], c["d"])

    def decode(self, x, past_len, rope_theta=0.0):
        import torch
        c = self.c
        B, _, D = x.shape
        xd = to_dev(x, c["dtype"])
        out = torch.empty((B, 1, c["Hq"] * c["d"]), dtype=torch_dtype(c["dtype"]), device="cuda")
        nb = self.dkv.workspace_bytes("decode", self.cache, B, 1, c["Hq"])
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.dkv.attn_decode(self.cache, xd, self.wq, self.wk, self.wv, past_len, c["Hq"], out, ws,
                             rope_theta=rope_theta)
        torch.cuda.synchronize()
        return from_dev(out).reshape(B, 1, c["Hq"], c["d"])

    def append(self, x, past_len):
        import torch
        xd = to_dev(x, self.c["dtype"])
        self.dkv.kv_append(self.cache, xd, self.wk, self.wv, past_len)
        torch.cuda.synchronize()

    def cache_k(self):
        return synth.from_storage(self.cache.k, self.c["dtype"])

    def cache_v(self):
        return synth.from_storage(self.cache.v, self.c["dtype"])

    def free(self):
        self.cache.free()


def oracle_step(case, x, past_len, kc, vc, t_index=None, rope_theta=0.0):
    """Oracle layer step on float32 cache copies (modified in place)."""
    return oracle.layer_step(x, case["wq"], case["wk"], case["wv"], kc, vc, past_len, case["Hq"],
                             case["dtype"], t_index=t_index, rope_theta=rope_theta)


def compare(got, ref, dtype, what=""):
    """Element-wise comparison against the fp64 oracle; returns (max_abs, mean_abs)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    tmax, tmean = TOL[dtype]
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e} (tol {tmax:g}/{tmean:g})", flush=True)
    assert mx <= tmax, f"{what}: max abs error {mx} > {tmax}"
    assert mean <= tmean, f"{what}: mean abs error {mean} > {tmean}"
    return mx, mean


def _ulp(a, dtype):
    """Spacing of `dtype` values at |a| (at least the smallest subnormal)."""
    p, emin = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** emin)))
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


def compare_rows(got, ref, dtype, absdot, D, what=""):
    """Appended cache rows against the oracle's: the GPU accumulates the D-term dot products
    in fp32 (error <= D * 2^-24 * sum|x||w|) and then rounds once to the cache dtype
    (<= 1 ulp here, allowing for the rounding boundary the fp32 error may cross).
    `absdot` holds sum_k |x_k||w_k| for every compared element."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = D * 2.0 ** -24 * np.asarray(absdot, dtype=np.float64) + _ulp(ref, dtype)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} appended values outside the fp32-accumulation bound"


def absdot_rows(x, w, Hkv, d):
    """sum_k |x[b,t,k]| |w[k, g*d+i]| arranged like cache rows: [B, Hkv, T, d]."""
    B, T, D = x.shape
    a = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w, np.float64))
    return a.reshape(B, T, Hkv, d).transpose(0, 2, 1, 3)
