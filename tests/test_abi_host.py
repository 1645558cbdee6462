"""C ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "directkv.h")
MAGIC = 0x444B5631   # the mark kv_alloc_host leaves in a descriptor


@pytest.fixture(scope="module")
def dkv():
    import zero_copy_host_amd as z
    if not os.path.exists(z.LIB_PATH):
        from zero_copy_host_amd import build
        build.build(verbose=False)
    z.lib()
    return z


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|int32_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function(dkv):
    declared = _declared_functions()
    assert {"kv_alloc_host", "kv_free_host", "kv_append", "attn_workspace_bytes", "attn_prefill",
            "attn_decode", "dkv_last_error"} <= set(declared)
    L = dkv.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(dkv.EXPORTS)
    assert dkv.version() >= 100


def _fake_cache(dkv, B=2, Hkv=2, d=128, cap=128, dtype=2):
    c = dkv.dkv_cache()
    c.k, c.v = 0x1000, 0x2000          # never dereferenced: every call below fails validation
    c.batch, c.n_kv_heads, c.head_dim, c.capacity, c.dtype, c.reserved = B, Hkv, d, cap, dtype, MAGIC
    return c


def _lens(vals):
    a = np.asarray(vals, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _err(dkv):
    return dkv.lib().dkv_last_error().decode()


def test_alloc_validation(dkv):
    L, c = dkv.lib(), dkv.dkv_cache()
    assert L.kv_alloc_host(None, 1, 1, 128, 64, 2) == -1
    assert L.kv_alloc_host(ctypes.byref(c), 0, 1, 128, 64, 2) == -1
    assert L.kv_alloc_host(ctypes.byref(c), 1, 1, 128, 100, 2) == -1
    assert "multiple of 64" in _err(dkv)
    assert L.kv_alloc_host(ctypes.byref(c), 1, 1, 96, 64, 2) == -3
    assert L.kv_alloc_host(ctypes.byref(c), 1, 1, 128, 64, 7) == -3
    assert c.k is None and c.reserved == 0
    assert L.kv_free_host(ctypes.byref(c)) == 0
    assert L.kv_free_host(None) == 0


def test_call_validation_statuses(dkv):
    L = dkv.lib()
    c = _fake_cache(dkv)
    x = w = out = ws = 0x10000
    lens, lp = _lens([10, 20])
    # capacity: 20 + 120 > 128
    assert L.attn_prefill(ctypes.byref(c), x, w, w, w, lp, 2, 120, 256, 4, out, ws, 1 << 30, None) == -2
    assert "capacity" in _err(dkv)
    neg, np_ = _lens([-1, 0])
    assert L.kv_append(ctypes.byref(c), x, w, w, np_, 2, 1, 256, None) == -2
    # batch mismatch, bad D, null and misaligned pointers
    assert L.kv_append(ctypes.byref(c), x, w, w, lp, 3, 1, 256, None) == -1
    assert L.kv_append(ctypes.byref(c), x, w, w, lp, 2, 1, 100, None) == -1
    assert L.kv_append(ctypes.byref(c), None, w, w, lp, 2, 1, 256, None) == -1
    assert L.kv_append(ctypes.byref(c), x + 4, w, w, lp, 2, 1, 256, None) == -1
    assert L.kv_append(ctypes.byref(c), x, w, w, None, 2, 1, 256, None) == -1
    # heads: Hq not a multiple of Hkv, unsupported group size
    assert L.attn_decode(ctypes.byref(c), x, w, w, w, lp, 2, 256, 3, out, ws, 1 << 30, None) == -1
    assert L.attn_decode(ctypes.byref(c), x, w, w, w, lp, 2, 256, 6, out, ws, 1 << 30, None) == -3
    # workspace too small
    assert L.attn_decode(ctypes.byref(c), x, w, w, w, lp, 2, 256, 4, out, ws, 16, None) == -6
    assert L.attn_prefill(ctypes.byref(c), x, w, w, w, lp, 2, 8, 256, 4, out, ws, 16, None) == -6
    # descriptor not made by kv_alloc_host
    bad = _fake_cache(dkv)
    bad.reserved = 0
    assert L.attn_decode(ctypes.byref(bad), x, w, w, w, lp, 2, 256, 4, out, ws, 1 << 30, None) == -1
    # unknown prefill / decode variant
    assert L.attn_prefill_variant(ctypes.byref(c), x, w, w, w, lp, 2, 8, 256, 4, out, ws, 1 << 30, None, 5) == -1
    assert L.attn_decode_variant(ctypes.byref(c), x, w, w, w, lp, 2, 256, 4, out, ws, 1 << 30, None, 2) == -1
    # the staging baselines check their larger workspace before any copy: what the zero-copy
    # call needs is too small for them
    plain_d = L.attn_workspace_bytes(1, ctypes.byref(c), 2, 1, 4, lp)
    plain_p = L.attn_workspace_bytes(0, ctypes.byref(c), 2, 8, 4, lp)
    assert L.attn_decode_variant(ctypes.byref(c), x, w, w, w, lp, 2, 256, 4, out, ws, plain_d, None, 1) == -6
    assert L.attn_prefill_variant(ctypes.byref(c), x, w, w, w, lp, 2, 8, 256, 4, out, ws, plain_p, None, 3) == -6
    assert L.kv_append(None, x, w, w, lp, 2, 1, 256, None) == -1
    # unsupported head_dim / dtype in a descriptor
    assert L.kv_append(ctypes.byref(_fake_cache(dkv, d=96)), x, w, w, lp, 2, 1, 256, None) == -3
    assert L.kv_append(ctypes.byref(_fake_cache(dkv, dtype=5)), x, w, w, lp, 2, 1, 256, None) == -3
    # more new K elements in one call than the kernels' 32-bit row indexing allows
    big = _fake_cache(dkv, B=2, Hkv=8, d=128, cap=1 << 30)
    bl, blp = _lens([0, 0])
    assert L.kv_append(ctypes.byref(big), x, w, w, blp, 2, 1 << 20, 256, None) == -3
    assert "2^31" in _err(dkv)
    # hostlink
    assert L.dkv_hostlink_stream(None, 1024, 0, 4, None) == -1
    assert L.dkv_hostlink_stream(0x1000, 1000, 0, 4, None) == -1
    assert L.dkv_hostlink_stream(0x1000, 1024, 2, 4, None) == -1


def test_batch_limit(dkv):
    """Lengths travel in kernel arguments: at most 256 sequences per call; more is UNSUPPORTED
    before anything is enqueued."""
    L = dkv.lib()
    c = _fake_cache(dkv, B=257)
    lens, lp = _lens([1] * 257)
    assert L.attn_decode(ctypes.byref(c), 0x10000, 0x10000, 0x10000, 0x10000, lp, 257, 256, 2,
                         0x10000, 0x10000, 1 << 30, None) == -3
    assert "257" in _err(dkv)
    assert L.kv_append(ctypes.byref(c), 0x10000, 0x10000, 0x10000, lp, 257, 1, 256, None) == -3


def test_zero_new_tokens_is_a_no_op(dkv):
    L = dkv.lib()
    c = _fake_cache(dkv)
    lens, lp = _lens([10, 20])
    # T = 0 passes validation and returns before any launch
    assert L.kv_append(ctypes.byref(c), 0x10000, 0x10000, 0x10000, lp, 2, 0, 256, None) == 0
    assert L.attn_prefill(ctypes.byref(c), 0x10000, 0x10000, 0x10000, 0x10000, lp, 2, 0, 256, 4,
                          0x10000, 0x10000, 1 << 30, None) == 0


def test_workspace_sizes(dkv):
    L = dkv.lib()
    c = _fake_cache(dkv, B=1, Hkv=8, d=128, cap=32768)
    lens, lp = _lens([24576])
    ws = L.attn_workspace_bytes(0, ctypes.byref(c), 1, 8192, 32, lp)
    e = 2
    # queries + new K + new V + two fp32 running states (past keys, this step's own keys): per 32
    # query rows, 64 lanes x (d/32 * 16 accumulators + m + l); then the rotary (cos, sin) fp32 table
    # of every new row's d/2 pairs
    state = 8 * (8192 * 4 // 32) * (4 * 16 + 2) * 64 * 4
    want = 8192 * 32 * 128 * e + 2 * 8 * 8192 * 128 * e + 2 * state
    want += 8192 * 64 * 2 * 4
    # the two-launch prefill: one more state per past super-chunk of 3072 keys (8 pairs, one per
    # XCD, 1.5 MiB of K and V each) for any past length up to capacity - T = 24576: 8 of them
    want += 8 * state
    assert want <= ws <= want + 7 * 256
    wsd = L.attn_workspace_bytes(1, ctypes.byref(c), 1, 1, 32, lp)
    # decode: fp32 partials (o, m, l) for at most 2 * (2 * 256 / Hkv) + B + 1 splits (the split
    # target doubles for short chunks), then the fp32 queries [B][Hq*d] the pre-pass projects
    def up(n):
        return (n + 255) // 256 * 256
    assert wsd == up((4 * 256 // 8 + 1 + 1) * 32 * (128 + 2) * 4) + up(1 * 32 * 128 * 4)
    # staging baselines: a device copy of the whole cache (K and V) on top
    staging = 2 * 1 * 8 * 32768 * 128 * e
    assert L.attn_workspace_bytes(2, ctypes.byref(c), 1, 8192, 32, lp) == staging + ws
    assert L.attn_workspace_bytes(3, ctypes.byref(c), 1, 1, 32, lp) == staging + wsd
    assert L.attn_workspace_bytes(4, ctypes.byref(c), 1, 1, 32, lp) == 0
    assert L.attn_workspace_bytes(1, None, 1, 1, 32, lp) == 0


def test_workspace_two_launch_prefill_region(dkv):
    """The super-chunk states of the two-launch prefill: present only where they fit 2 GiB and the
    call has more than one query tile per pair and more than one super-chunk of past keys."""
    L = dkv.lib()
    lens, lp = _lens([0, 0])

    def up(n):
        return (n + 255) // 256 * 256

    def ws(B, Hkv, cap, T, Hq):
        c = _fake_cache(dkv, B=B, Hkv=Hkv, d=128, cap=cap)
        return L.attn_workspace_bytes(0, ctypes.byref(c), B, T, Hq, lp)

    def state(B, Hkv, T, G):
        return up(B * Hkv * (T * G // 32) * (4 * 16 + 2) * 64 * 4)

    def base(B, Hkv, T, Hq):   # queries, new K and V, two running states, rotary table (bf16, d = 128)
        G = Hq // Hkv
        return (up(B * T * Hq * 128 * 2) + 2 * up(B * Hkv * T * 128 * 2) + 2 * state(B, Hkv, T, G)
                + up(B * T * 64 * 2 * 4))

    # 70B-shaped (B=2, Hkv=8, G=8, T=16384, capacity 65600): 17 super-chunks x 1.09 GB is over the
    # cap, so the launch-per-super-chunk path runs and there is no region
    assert ws(2, 8, 65600, 16384, 64) == base(2, 8, 16384, 64)
    # at most one super-chunk of 3072 past keys: no region
    assert ws(1, 8, 8192 + 3072, 8192, 32) == base(1, 8, 8192, 32)
    # two super-chunks: two states
    assert ws(1, 8, 8192 + 3073, 8192, 32) == base(1, 8, 8192, 32) + 2 * state(1, 8, 8192, 4)


def test_workspace_without_two_launch_prefill(dkv, monkeypatch):
    """DIRECTKV_PREFILL_CHUNKED=0 keeps the launch-per-super-chunk path and the workspace query
    then leaves the super-chunk states out (the 8B-shaped prefill: 1.49 GB -> 382 MB)."""
    L = dkv.lib()
    c = _fake_cache(dkv, B=1, Hkv=8, d=128, cap=32768)
    lens, lp = _lens([24576])
    with_states = L.attn_workspace_bytes(0, ctypes.byref(c), 1, 8192, 32, lp)
    monkeypatch.setenv("DIRECTKV_PREFILL_CHUNKED", "0")
    without = L.attn_workspace_bytes(0, ctypes.byref(c), 1, 8192, 32, lp)
    state = 8 * (8192 * 4 // 32) * (4 * 16 + 2) * 64 * 4
    assert with_states - without == 8 * state
    assert without < 400 * 10 ** 6


# ---- paged cache: the block table is checked on the host before anything is enqueued

PAGED_MAGIC = 0x444B5650   # the mark kv_paged_alloc_host leaves in a descriptor


def _fake_paged(dkv, n_pages=8, Hkv=2, d=128, dtype=2):
    c = dkv.dkv_paged_cache()
    c.k, c.v = 0x1000, 0x2000          # never dereferenced: every call below stops before a launch
    c.n_pages, c.n_kv_heads, c.head_dim, c.dtype, c.reserved = n_pages, Hkv, d, dtype, PAGED_MAGIC
    return c


def _tab(rows):
    t = np.ascontiguousarray(np.array(rows, dtype=np.int32))
    return t, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), t.shape[1]


def test_paged_alloc_validation(dkv):
    L, pc = dkv.lib(), dkv.dkv_paged_cache()
    assert L.kv_paged_alloc_host(None, 4, 2, 128, 2) == -1
    assert L.kv_paged_alloc_host(ctypes.byref(pc), 0, 2, 128, 2) == -1
    assert L.kv_paged_alloc_host(ctypes.byref(pc), 4, 2, 96, 2) == -3
    # a pool whose byte count overflows is refused before any allocation
    assert L.kv_paged_alloc_host(ctypes.byref(pc), 2**31 - 1, 2**31 - 1, 128, 0) == -1
    assert "overflows" in _err(dkv)
    assert pc.k is None and pc.reserved == 0


def test_paged_table_validation(dkv):
    L = dkv.lib()
    c = _fake_paged(dkv)
    x = w = out = ws = 0x10000
    big = 1 << 30
    lens, lp = _lens([20, 3])                       # sequence 0 uses pages 0-1, sequence 1 page 0
    ok, okp, mp = _tab([[4, 5, -1], [6, -1, -1]])
    # a valid table gets through every check; T = 0 then returns before any copy or launch
    assert L.attn_prefill_paged(ctypes.byref(c), okp, mp, x, w, w, w, lp, 2, 0, 256, 8, out, ws, big, None) == 0
    # page id outside the pool
    bad, badp, _ = _tab([[4, 9, -1], [6, -1, -1]])
    assert L.attn_decode_paged(ctypes.byref(c), badp, mp, x, w, w, w, lp, 2, 256, 8, out, ws, big, None) == -1
    assert "outside" in _err(dkv)
    # an unused entry (-1) beyond the used pages is fine; a used -1 is not
    bad, badp, _ = _tab([[4, -1, -1], [6, -1, -1]])
    assert L.attn_decode_paged(ctypes.byref(c), badp, mp, x, w, w, w, lp, 2, 256, 8, out, ws, big, None) == -1
    # the page a call writes may not be mapped twice (sequence 1 writes token 3 on page 4,
    # which sequence 0 also reads)
    bad, badp, _ = _tab([[4, 5, -1], [4, -1, -1]])
    assert L.attn_decode_paged(ctypes.byref(c), badp, mp, x, w, w, w, lp, 2, 256, 8, out, ws, big, None) == -1
    assert "mapped 2 times" in _err(dkv)
    # shared pages that nobody writes are fine: both read page 4, sequence 1 writes page 7
    lens2, lp2 = _lens([20, 16])
    sh, shp, _ = _tab([[4, 5, -1], [4, 7, -1]])
    assert L.attn_prefill_paged(ctypes.byref(c), shp, mp, x, w, w, w, lp2, 2, 0, 256, 8, out, ws, big, None) == 0
    # capacity: 3 pages hold 48 tokens
    lens3, lp3 = _lens([47, 0])
    assert L.attn_decode_paged(ctypes.byref(c), okp, mp, x, w, w, w, lp3, 2, 256, 8, out, ws, big, None) in (-1, -2)
    lens4, lp4 = _lens([48, 0])
    full, fullp, _ = _tab([[0, 1, 2], [3, -1, -1]])
    assert L.attn_decode_paged(ctypes.byref(c), fullp, mp, x, w, w, w, lp4, 2, 256, 8, out, ws, big, None) == -2
    # workspace too small, null table, descriptor not from kv_paged_alloc_host
    assert L.attn_decode_paged(ctypes.byref(c), okp, mp, x, w, w, w, lp, 2, 256, 8, out, ws, 64, None) == -6
    assert L.kv_paged_append(ctypes.byref(c), okp, mp, x, w, w, lp, 2, 1, 256, ws, 16, None) == -6
    assert L.attn_decode_paged(ctypes.byref(c), None, mp, x, w, w, w, lp, 2, 256, 8, out, ws, big, None) == -1
    nd = _fake_paged(dkv)
    nd.reserved = MAGIC                              # a contiguous descriptor's mark
    assert L.attn_decode_paged(ctypes.byref(nd), okp, mp, x, w, w, w, lp, 2, 256, 8, out, ws, big, None) == -1


def test_paged_workspace_sizes(dkv):
    L = dkv.lib()
    c = _fake_paged(dkv, n_pages=4096, Hkv=8)
    cc = _fake_cache(dkv, B=2, Hkv=8, d=128, cap=64 * 16)
    lens, lp = _lens([500, 900])
    table_bytes = ((2 * 64 * 4 + 255) // 256) * 256
    assert L.attn_paged_workspace_bytes(2, ctypes.byref(c), 2, 1, 32, 64) == table_bytes
    # prefill: the table plus exactly what the contiguous call needs
    assert (L.attn_paged_workspace_bytes(0, ctypes.byref(c), 2, 128, 32, 64)
            == table_bytes + L.attn_workspace_bytes(0, ctypes.byref(cc), 2, 128, 32, lp))
    # decode: the table plus at least the contiguous partials
    assert (L.attn_paged_workspace_bytes(1, ctypes.byref(c), 2, 1, 32, 64)
            >= table_bytes + L.attn_workspace_bytes(1, ctypes.byref(cc), 2, 1, 32, lp))
    assert L.attn_paged_workspace_bytes(1, None, 2, 1, 32, 64) == 0
    assert L.attn_paged_workspace_bytes(1, ctypes.byref(c), 2, 1, 32, 0) == 0


def test_disabled_persistent_prefill_is_refused_before_any_launch(dkv):
    L = dkv.lib()
    c = _fake_cache(dkv, B=1, Hkv=8, d=128, cap=4096)
    lens, lp = _lens([1000])
    x = w = out = ws = 0x10000
    assert L.attn_prefill_variant(ctypes.byref(c), x, w, w, w, lp, 1, 64, 256, 32, out, ws, 1 << 30, None, 4) == -3
    assert "disabled" in _err(dkv)


# ---- the Python binding refuses unusable tensors before any library call

def _fake_host_cache(dkv, B=2, Hkv=2, d=128, cap=128, dtype="bf16", live=True):
    import types
    c = _fake_cache(dkv, B=B, Hkv=Hkv, d=d, cap=cap, dtype=dkv.DTYPE_CODES[dtype])
    if not live:
        c.reserved = 0
    return types.SimpleNamespace(desc=c, dtype=dtype, shape=(B, Hkv, cap, d))


def _layer_tensors(B=2, T=8, D=256, Hq=4, Hkv=2, d=128, dtype=None):
    import torch
    dt = dtype or torch.bfloat16
    return dict(x=torch.zeros(B, T, D, dtype=dt), wq=torch.zeros(Hq * d, D, dtype=dt),
                wk=torch.zeros(Hkv * d, D, dtype=dt), wv=torch.zeros(Hkv * d, D, dtype=dt),
                out=torch.zeros(B, T, Hq * d, dtype=dt), ws=torch.zeros(1024, dtype=torch.uint8))


def _prefill(dkv, cache, t, Hq=4):
    dkv.attn_prefill(cache, t["x"], t["wq"], t["wk"], t["wv"], [0, 0], Hq, t["out"], t["ws"])


def test_binding_refuses_host_tensors(dkv):
    """Tensors in host memory would make the kernels read pageable memory: refused."""
    cache = _fake_host_cache(dkv)
    t = _layer_tensors()
    with pytest.raises(ValueError, match="must be a device"):
        _prefill(dkv, cache, t)
    with pytest.raises(ValueError, match="must be a device"):
        dkv.attn_decode(cache, t["x"][:, :1].contiguous(), t["wq"], t["wk"], t["wv"], [0, 0], 4,
                        t["out"][:, :1].contiguous(), t["ws"])
    with pytest.raises(ValueError, match="must be a device"):
        dkv.kv_append(cache, t["x"], t["wk"], t["wv"], [0, 0])


def test_binding_refuses_wrong_dtype_shape_layout(dkv):
    import torch
    cache = _fake_host_cache(dkv)
    t = _layer_tensors()
    bad = dict(t, x=t["x"].float())                              # f32 activations, bf16 cache
    with pytest.raises(ValueError, match="dtype"):
        _prefill(dkv, cache, bad)
    bad = dict(t, wk=torch.zeros(2 * 128, 128, dtype=torch.bfloat16))   # wrong reduction width
    with pytest.raises(ValueError, match="shape"):
        _prefill(dkv, cache, bad)
    bad = dict(t, wq=torch.zeros(256, 4 * 128, dtype=torch.bfloat16).t())   # a transposed view
    with pytest.raises(ValueError, match="contiguous"):
        _prefill(dkv, cache, bad)
    bad = dict(t, out=torch.zeros(2, 7, 512, dtype=torch.bfloat16))   # too small for T = 8
    with pytest.raises(ValueError, match="elements"):
        _prefill(dkv, cache, bad)
    bad = dict(t, ws=[0] * 16)
    with pytest.raises(TypeError, match="torch tensor"):
        _prefill(dkv, cache, bad)
    with pytest.raises(ValueError, match="live cache"):
        _prefill(dkv, _fake_host_cache(dkv, live=False), t)
    with pytest.raises(ValueError, match="live cache"):
        _prefill(dkv, object(), t)


def test_binding_refuses_bad_decode_loop_tensors(dkv):
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be a device"):
        dkv.rmsnorm(x, torch.zeros(256, dtype=torch.bfloat16), x)
    with pytest.raises(ValueError, match="shape"):
        dkv.rmsnorm(x, torch.zeros(128, dtype=torch.bfloat16), x)
    with pytest.raises(ValueError, match="dtype"):
        dkv.linear(x, torch.zeros(64, 256, dtype=torch.float16), torch.zeros(4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="elements"):
        dkv.linear(x, torch.zeros(64, 256, dtype=torch.bfloat16), torch.zeros(4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be a device"):
        dkv.swiglu(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="unsupported dtype"):
        dkv.swiglu(torch.zeros(4, 64, dtype=torch.int32), torch.zeros(4, 32, dtype=torch.int32))


def test_rope_base_validation(dkv):
    """attn_prefill_rope / attn_decode_rope take a finite rotary base above 1; anything else is
    INVALID_ARG before any workspace, memory or HIP check."""
    L = dkv.lib()
    c = _fake_cache(dkv, B=2, Hkv=2, d=128, cap=4096)
    x = w = out = ws = 0x10000
    lens, lp = _lens([10, 20])
    for theta in (0.0, 1.0, 0.5, -10000.0, float("nan"), float("inf"), 1e31):
        assert L.attn_prefill_rope(ctypes.byref(c), x, w, w, w, lp, 2, 16, 256, 8, out, ws, 1 << 30, theta,
                                   None) == -1, theta
        assert "rope_theta" in _err(dkv)
        assert L.attn_decode_rope(ctypes.byref(c), x, w, w, w, lp, 2, 256, 8, out, ws, 1 << 30, theta, None) == -1
        assert "rope_theta" in _err(dkv)
    # a good base goes on to the next check (here: the workspace is too small)
    assert L.attn_prefill_rope(ctypes.byref(c), x, w, w, w, lp, 2, 16, 256, 8, out, ws, 16, 500000.0, None) == -6
    assert L.attn_decode_rope(ctypes.byref(c), x, w, w, w, lp, 2, 256, 8, out, ws, 16, 10000.0, None) == -6
    # the usual argument checks come first
    assert L.attn_prefill_rope(ctypes.byref(c), x, w, w, w, lp, 2, 16, 256, 7, out, ws, 1 << 30, 500000.0,
                               None) == -1
    assert "rope_theta" not in _err(dkv)


def test_key_split_workspace_follows_the_pair_count(dkv):
    """A prefill with one query tile per pair (T * G <= 256) reserves running states for its key
    splits: 32 per pair with few pairs, fewer as pairs grow, none from 512 pairs on."""
    L = dkv.lib()
    r256 = lambda n: -(-n // 256) * 256
    d, e, Hkv, Hq = 128, 2, 8, 32

    def ws(B, T):
        c = _fake_cache(dkv, B=B, Hkv=Hkv, d=d, cap=4096)
        lens, lp = _lens([1000] * B)
        return L.attn_workspace_bytes(0, ctypes.byref(c), B, T, Hq, lp)

    def expected(B, T, splits):
        G = Hq // Hkv
        state = r256(B * Hkv * (-(-(T * G) // 32)) * (d // 32 * 16 + 2) * 64 * 4)
        return (r256(B * T * Hq * d * e) + 2 * r256(B * Hkv * T * d * e) + 2 * state
                + r256(B * T * (d // 2) * 2 * 4) + splits * state)

    # 512 query rows per pair: two tiles, no key splits; the two-launch prefill's states instead, one
    # per super-chunk of 3072 keys for past lengths up to 4096 - 128
    assert ws(1, 128) == expected(1, 128, 2)
    assert ws(1, 16) == expected(1, 16, 32)       # 8 pairs: 32 splits each
    assert ws(8, 16) == expected(8, 16, 8)        # 64 pairs: 8
    assert ws(64, 16) == expected(64, 16, 0)      # 512 pairs: one split each, none reserved
