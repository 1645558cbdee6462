"""Paged host cache (16-token pages + block table) through the C ABI.

The paged calls must compute exactly what the contiguous calls compute on the same logical
cache: same kernels, same plan, only the row addressing differs. So besides the oracle
tolerance, outputs and appended rows are compared bit for bit with the contiguous path on
the same inputs, and pages the call must not touch keep their NaN canaries.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import GpuLayer, compare, fill_canary, oracle_step, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

PT = 16


def _case(seed, B, T, past, D, Hq, Hkv, d, dtype):
    cap = ((max(past) + T + 63) // 64 + 1) * 64
    return synth.draw_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap)


class PagedLayer:
    """A page pool holding the case's past K/V through a shuffled block table, plus device
    weights. `share` > 0 maps the first `share` logical pages of every sequence to the pages
    of sequence 0 (a shared prefix, read only; the case must have equal prefixes there)."""

    def __init__(self, case, seed=0, spare=5, share=0):
        import zero_copy_host_amd as dkv
        self.dkv, self.c = dkv, case
        c = case
        dt = c["dtype"]
        need = [(int(L) + c["T"] + PT - 1) // PT for L in c["past_len"]]
        self.max_pages = max(need) + 1
        n_pages = sum(need) + spare
        self.cache = dkv.PagedHostKVCache(n_pages, c["Hkv"], c["d"], dt)
        fill_canary(self.cache.k, dt)
        fill_canary(self.cache.v, dt)
        rng = np.random.default_rng(seed)
        free = list(rng.permutation(n_pages))
        lists = []
        for b, n in enumerate(need):
            own = [int(free.pop()) for _ in range(n - (share if b else 0))]
            lists.append((lists[0][:share] + own) if b and share else own)
        self.table = dkv.block_table(lists, self.max_pages)
        for b in range(c["B"]):
            L = int(c["past_len"][b])
            for j in range(L):
                pg, r = self.table[b, j // PT], j % PT
                self.cache.k[pg, :, r] = synth.to_storage(c["kp"][b, :, j], dt)
                self.cache.v[pg, :, r] = synth.to_storage(c["vp"][b, :, j], dt)
        self.wq = to_dev(c["wq"].T, dt)
        self.wk = to_dev(c["wk"].T, dt)
        self.wv = to_dev(c["wv"].T, dt)

    def _ws(self, phase, B, T):
        import torch
        nb = self.dkv.paged_workspace_bytes(phase, self.cache, B, T, self.c["Hq"], self.max_pages)
        assert nb > 0
        return torch.empty(nb, dtype=torch.uint8, device="cuda")

    def decode(self, x, past_len):
        import torch
        c = self.c
        B = x.shape[0]
        out = torch.empty((B, 1, c["Hq"] * c["d"]), dtype=torch_dtype(c["dtype"]), device="cuda")
        self.dkv.attn_decode_paged(self.cache, self.table, to_dev(x, c["dtype"]), self.wq, self.wk, self.wv,
                                   past_len, c["Hq"], out, self._ws("decode", B, 1))
        torch.cuda.synchronize()
        return out.float().cpu().numpy().reshape(B, 1, c["Hq"], c["d"])

    def prefill(self, x, past_len):
        import torch
        c = self.c
        B, T, _ = x.shape
        out = torch.empty((B, T, c["Hq"] * c["d"]), dtype=torch_dtype(c["dtype"]), device="cuda")
        self.dkv.attn_prefill_paged(self.cache, self.table, to_dev(x, c["dtype"]), self.wq, self.wk, self.wv,
                                    past_len, c["Hq"], out, self._ws("prefill", B, T))
        torch.cuda.synchronize()
        return out.float().cpu().numpy().reshape(B, T, c["Hq"], c["d"])

    def append(self, x, past_len):
        import torch
        c = self.c
        B, T, _ = x.shape
        self.dkv.kv_paged_append(self.cache, self.table, to_dev(x, c["dtype"]), self.wk, self.wv, past_len,
                                 self._ws("append", B, T))
        torch.cuda.synchronize()

    def logical_bits(self, pool, n_tokens):
        """Storage bits of the logical cache rows [B][Hkv][n][d] (gathered through the table)."""
        c = self.c
        out = np.zeros((c["B"], c["Hkv"], n_tokens, c["d"]), dtype=pool.dtype)
        for b in range(c["B"]):
            for j in range(n_tokens):
                out[b, :, j] = pool[self.table[b, j // PT], :, j % PT]
        return out

    def touched_pages(self, past_len, T):
        pages = set()
        for b in range(self.c["B"]):
            L = int(past_len[b])
            pages.update(int(self.table[b, j // PT]) for j in range(0, L + T))
        return pages

    def free(self):
        self.cache.free()


def _contiguous(case, fn):
    g = GpuLayer(case)
    try:
        out = fn(g)
        return out, g.cache.k.copy(), g.cache.v.copy()
    finally:
        g.free()


def _check_untouched(pl, past_len, T):
    """Pages outside the used part of the table still hold the canaries."""
    used = pl.touched_pages(past_len, T)
    for p in range(pl.cache.n_pages):
        if p not in used:
            k, v = pl.cache.k[p], pl.cache.v[p]
            if pl.c["dtype"] == "f32":
                assert np.isnan(k).all() and np.isnan(v).all(), f"page {p} was written"
            else:
                nan = np.uint16(0x7FC1 if pl.c["dtype"] == "bf16" else 0x7E01)
                assert (k == nan).all() and (v == nan).all(), f"page {p} was written"


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f16", 64, 2), ("f32", 64, 1)])
def test_paged_decode_equals_contiguous_bitwise(dtype, d, G):
    Hkv = 2
    case = _case(301, 3, 1, [100, 37, 250], 256, Hkv * G, Hkv, d, dtype)
    x, past = case["x"], case["past_len"]
    out_c, kc_bits, vc_bits = _contiguous(case, lambda g: g.decode(x, past))
    pl = PagedLayer(case, seed=1)
    try:
        out_p = pl.decode(x, past)
        n = int(max(past)) + 1
        kp_bits, vp_bits = pl.logical_bits(pl.cache.k, n), pl.logical_bits(pl.cache.v, n)
        _check_untouched(pl, past, 1)
    finally:
        pl.free()
    assert np.array_equal(out_p, out_c), "paged decode differs from contiguous decode"
    for b in range(case["B"]):
        L = int(past[b])
        assert np.array_equal(kp_bits[b, :, : L + 1], kc_bits[b, :, : L + 1])
        assert np.array_equal(vp_bits[b, :, : L + 1], vc_bits[b, :, : L + 1])
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, x, past, kc, vc)
    compare(out_p, ref, dtype, f"paged decode {dtype} d{d} G{G}")


@pytest.mark.parametrize("chunk,two_launch", [(None, "0"), ("64", "0"), ("64", "1")])
def test_paged_prefill_equals_contiguous_bitwise(chunk, two_launch, monkeypatch):
    """Several super-chunks (chunk 64: many launches, the new rows stored by several of
    them), ragged query tiles, two sequences of different lengths; with the launch-per-super-chunk
    path and with the two-launch form (three super-chunk states merged at the end), both caches
    held to the same path and super-chunk size."""
    monkeypatch.setenv("DIRECTKV_PREFILL_CHUNKED", two_launch)
    if chunk:
        monkeypatch.setenv("DIRECTKV_PREFILL_CHUNK", chunk)
    case = _case(302, 2, 70, [33, 130], 256, 8, 2, 128, "bf16")
    x, past = case["x"], case["past_len"]
    out_c, kc_bits, vc_bits = _contiguous(case, lambda g: g.prefill(x, past))
    pl = PagedLayer(case, seed=2)
    try:
        out_p = pl.prefill(x, past)
        n = int(max(past)) + case["T"]
        kp_bits, vp_bits = pl.logical_bits(pl.cache.k, n), pl.logical_bits(pl.cache.v, n)
        _check_untouched(pl, past, case["T"])
    finally:
        pl.free()
    assert np.array_equal(out_p, out_c), "paged prefill differs from contiguous prefill"
    for b in range(case["B"]):
        m = int(past[b]) + case["T"]
        assert np.array_equal(kp_bits[b, :, :m], kc_bits[b, :, :m])
        assert np.array_equal(vp_bits[b, :, :m], vc_bits[b, :, :m])
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, x, past, kc, vc)
    compare(out_p, ref, "bf16", f"paged prefill chunk={chunk}")


def test_paged_key_split_prefill_equals_contiguous_bitwise():
    """One query tile per pair, so the keys are split over workgroups; a past of 20000 keys is
    longer than one paged launch may stage, so the splits are also bounded by that."""
    case = _case(303, 2, 16, [20000, 5000], 256, 8, 2, 128, "bf16")
    x, past = case["x"], case["past_len"]
    out_c, kc_bits, vc_bits = _contiguous(case, lambda g: g.prefill(x, past))
    pl = PagedLayer(case, seed=3)
    try:
        out_p = pl.prefill(x, past)
        n = int(max(past)) + case["T"]
        kp_bits, vp_bits = pl.logical_bits(pl.cache.k, n), pl.logical_bits(pl.cache.v, n)
        _check_untouched(pl, past, case["T"])
    finally:
        pl.free()
    assert np.array_equal(out_p, out_c), "paged prefill differs from contiguous prefill"
    for b in range(case["B"]):
        m = int(past[b]) + case["T"]
        assert np.array_equal(kp_bits[b, :, :m], kc_bits[b, :, :m])
        assert np.array_equal(vp_bits[b, :, :m], vc_bits[b, :, :m])
    kc, vc = case["kp"].copy(), case["vp"].copy()
    compare(out_p, oracle_step(case, x, past, kc, vc), "bf16", "paged prefill with key splits")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_append_equals_contiguous_bitwise(dtype):
    case = _case(303, 3, 37, [5, 0, 130], 256, 4, 2, 64, dtype)
    x, past = case["x"], case["past_len"]
    _, kc_bits, vc_bits = _contiguous(case, lambda g: g.append(x, past))
    pl = PagedLayer(case, seed=3)
    try:
        pl.append(x, past)
        n = int(max(past)) + case["T"]
        kp_bits, vp_bits = pl.logical_bits(pl.cache.k, n), pl.logical_bits(pl.cache.v, n)
        _check_untouched(pl, past, case["T"])
    finally:
        pl.free()
    for b in range(case["B"]):
        m = int(past[b]) + case["T"]
        assert np.array_equal(kp_bits[b, :, :m], kc_bits[b, :, :m])
        assert np.array_equal(vp_bits[b, :, :m], vc_bits[b, :, :m])


def test_paged_decode_with_a_shared_prefix():
    """Sequences 1 and 2 map their first 3 logical pages to sequence 0's pages (a shared
    48-token prefix, read only); each then appends its own token on a page of its own."""
    case = _case(304, 3, 1, [60, 75, 50], 256, 8, 2, 128, "bf16")
    for b in (1, 2):   # equal prefixes, as a shared page implies
        case["kp"][b, :, :48] = case["kp"][0, :, :48]
        case["vp"][b, :, :48] = case["vp"][0, :, :48]
    x, past = case["x"], case["past_len"]
    pl = PagedLayer(case, seed=4, share=3)
    try:
        assert (pl.table[1, :3] == pl.table[0, :3]).all() and (pl.table[2, :3] == pl.table[0, :3]).all()
        out = pl.decode(x, past)
    finally:
        pl.free()
    kc, vc = case["kp"].copy(), case["vp"].copy()
    ref = oracle_step(case, x, past, kc, vc)
    compare(out, ref, "bf16", "paged decode, shared prefix")


def test_paged_calls_reject_bad_tables_and_enqueue_nothing():
    import torch
    import zero_copy_host_amd as dkv
    case = _case(305, 2, 1, [40, 20], 256, 8, 2, 128, "bf16")
    x, past = case["x"], case["past_len"]
    pl = PagedLayer(case, seed=5, spare=2)
    try:
        before_k, before_v = pl.cache.k.copy(), pl.cache.v.copy()
        good = pl.table.copy()
        xd = to_dev(x, "bf16")
        out = torch.zeros((2, 1, 8 * 128), dtype=torch.bfloat16, device="cuda")
        ws = pl._ws("decode", 2, 1)

        def call(table, wsb=ws):
            return pl.dkv.lib().attn_decode_paged(
                __import__("ctypes").byref(pl.cache.desc),
                np.ascontiguousarray(table, dtype=np.int32).ctypes.data_as(
                    __import__("ctypes").POINTER(__import__("ctypes").c_int32)),
                table.shape[1], xd.data_ptr(), pl.wq.data_ptr(), pl.wk.data_ptr(), pl.wv.data_ptr(),
                np.ascontiguousarray(past, dtype=np.int32).ctypes.data_as(
                    __import__("ctypes").POINTER(__import__("ctypes").c_int32)),
                2, 256, 8, out.data_ptr(), wsb.data_ptr(), wsb.numel(), None)

        bad = good.copy()
        bad[1, 0] = pl.cache.n_pages           # page id out of range
        assert call(bad) == -1 and "outside" in dkv.lib().dkv_last_error().decode()
        bad = good.copy()
        bad[1, 1] = good[0, 2]                  # sequence 1 writes a page sequence 0 also maps
        assert call(bad) == -1 and "mapped" in dkv.lib().dkv_last_error().decode()
        small = torch.empty(64, dtype=torch.uint8, device="cuda")
        assert call(good, small) == -6
        torch.cuda.synchronize()
        assert np.array_equal(pl.cache.k, before_k) and np.array_equal(pl.cache.v, before_v)
        assert not out.any().item()
    finally:
        pl.free()


def test_paged_pool_holds_no_device_memory_and_reports_host_bytes():
    import torch
    import zero_copy_host_amd as dkv
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    pool = dkv.PagedHostKVCache(4096, 8, 128, "bf16")   # 4096 pages x 64 KiB = 256 MiB of host memory
    try:
        st = pool.memory_stats()
        assert st["host_bytes_total"] == 4096 * 2 * 8 * 16 * 128 * 2 and st["device_bytes"] == 0
        pages = pool.allocate(100)
        assert len(set(pages)) == 100 and pool.memory_stats()["pages_used"] == 100
        pool.release(pages)
        assert pool.memory_stats()["pages_used"] == 0
        assert torch.cuda.memory_allocated() == before
        assert torch.cuda.mem_get_info()[0] >= free0 - (64 << 20)
    finally:
        pool.free()
