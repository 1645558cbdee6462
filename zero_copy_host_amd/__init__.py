"""Python binding of libdirectkv.so: a host-resident KV-cache attention layer for MI355X.

Thin ctypes marshalling over the C ABI declared in include/directkv.h. All of the layer's
arithmetic runs in the HIP kernels of the library; this module only checks argument
shapes and passes device pointers, the host cache descriptor and the current HIP stream.
PyTorch supplies device memory and streams. There is no fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libdirectkv.so")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "CAPACITY", -3: "UNSUPPORTED", -4: "HOST_ALLOC",
          -5: "HIP", -6: "WORKSPACE"}
EXPORTS = ("kv_alloc_host", "kv_free_host", "kv_append", "attn_workspace_bytes", "attn_prefill",
           "attn_prefill_variant", "attn_decode", "attn_decode_variant", "attn_decode_noalloc", "attn_prefill_rope",
           "attn_decode_rope", "kv_paged_alloc_host", "kv_paged_free_host",
           "attn_paged_workspace_bytes", "kv_paged_append", "attn_prefill_paged", "attn_decode_paged",
           "dkv_rmsnorm", "dkv_linear", "dkv_swiglu", "dkv_hostlink_stream", "dkv_timing", "dkv_timing_read",
           "dkv_last_error", "dkv_version")
PAGE_TOKENS = 16
PREFILL_VARIANTS = {"fused": 0, "naive": 1, "separate": 2, "staged": 3, "persistent": 4}
DECODE_VARIANTS = {"zerocopy": 0, "staged": 1}


class DirectKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)} ({status}): {message}")
        self.status = status


class dkv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class dkv_paged_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_pages", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("pad", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m zero_copy_host_amd.build` first")
        # PyTorch ships its own HIP runtime. Loading torch first makes the library's
        # libamdhip64.so.7 / libhsa-runtime64.so.1 dependencies bind to those copies, so the
        # process holds one HIP runtime shared by torch tensors, streams and our kernels.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        L.kv_alloc_host.argtypes = [P(dkv_cache), I32, I32, I32, I32, I32]
        L.kv_free_host.argtypes = [P(dkv_cache)]
        L.kv_append.argtypes = [P(dkv_cache), VP, VP, VP, P(I32), I32, I32, I32, VP]
        L.attn_workspace_bytes.argtypes = [I32, P(dkv_cache), I32, I32, I32, P(I32)]
        L.attn_workspace_bytes.restype = SZ
        L.attn_prefill.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, I32, VP, VP, SZ, VP]
        L.attn_prefill_variant.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, I32, VP, VP, SZ,
                                           VP, I32]
        L.attn_decode.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, VP, VP, SZ, VP]
        L.attn_decode_variant.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, VP, VP, SZ, VP, I32]
        L.attn_decode_noalloc.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, VP, VP]
        D64 = ctypes.c_double
        L.attn_prefill_rope.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, I32, VP, VP, SZ, D64, VP]
        L.attn_decode_rope.argtypes = [P(dkv_cache), VP, VP, VP, VP, P(I32), I32, I32, I32, VP, VP, SZ, D64, VP]
        L.kv_paged_alloc_host.argtypes = [P(dkv_paged_cache), I32, I32, I32, I32]
        L.kv_paged_free_host.argtypes = [P(dkv_paged_cache)]
        L.attn_paged_workspace_bytes.argtypes = [I32, P(dkv_paged_cache), I32, I32, I32, I32]
        L.attn_paged_workspace_bytes.restype = SZ
        L.kv_paged_append.argtypes = [P(dkv_paged_cache), P(I32), I32, VP, VP, VP, P(I32), I32, I32, I32, VP, SZ, VP]
        L.attn_prefill_paged.argtypes = [P(dkv_paged_cache), P(I32), I32, VP, VP, VP, VP, P(I32), I32, I32, I32,
                                         I32, VP, VP, SZ, VP]
        L.attn_decode_paged.argtypes = [P(dkv_paged_cache), P(I32), I32, VP, VP, VP, VP, P(I32), I32, I32, I32,
                                        VP, VP, SZ, VP]
        L.dkv_rmsnorm.argtypes = [VP, VP, VP, I32, I32, ctypes.c_float, I32, VP]
        L.dkv_linear.argtypes = [VP, VP, VP, VP, I32, I32, I32, I32, VP]
        L.dkv_swiglu.argtypes = [VP, VP, I32, I32, I32, VP]
        L.dkv_hostlink_stream.argtypes = [VP, SZ, I32, I32, VP]
        L.dkv_timing.argtypes = [I32]
        L.dkv_timing_read.argtypes = [P(ctypes.c_float), P(I32), I32]
        L.dkv_last_error.restype = ctypes.c_char_p
        L.dkv_version.restype = I32
        for name in ("kv_alloc_host", "kv_free_host", "kv_append", "attn_prefill", "attn_prefill_variant",
                     "attn_decode", "attn_decode_variant", "attn_decode_noalloc", "attn_prefill_rope", "attn_decode_rope",
                     "kv_paged_alloc_host", "kv_paged_free_host", "kv_paged_append",
                     "attn_prefill_paged", "attn_decode_paged", "dkv_rmsnorm", "dkv_linear", "dkv_swiglu",
                     "dkv_hostlink_stream", "dkv_timing", "dkv_timing_read"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise DirectKVError(status, lib().dkv_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


_CODE_NAMES = {v: k for k, v in DTYPE_CODES.items()}


def _torch_code(t) -> Optional[int]:
    import torch
    return {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}.get(t.dtype)


def _tensor(t, name: str, code: Optional[int] = None, shape=None, numel: Optional[int] = None,
            device: bool = True):
    """Refuse, before any library call, a tensor the kernels could not use safely: not a
    torch tensor, not contiguous, of another dtype than the call's, of the wrong shape or size,
    or (device=True) not in device memory (the kernels would read pageable host memory or out of
    bounds)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if code is not None and _torch_code(t) != code:
        raise ValueError(f"{name} has dtype {t.dtype}; this call computes in {_CODE_NAMES[code]}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()} (shape {tuple(t.shape)})")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor, got one on {t.device}")
    return t


def _tensors(*specs) -> None:
    """_tensor over several (tensor, name, kwargs) specs: every layout check first, then the
    placement of each, so that the message names the first real mismatch."""
    for t, name, kw in specs:
        _tensor(t, name, device=False, **kw)
    for t, name, kw in specs:
        _tensor(t, name, **kw)


def _cache_desc(cache, kind):
    """The live descriptor of a HostKVCache / PagedHostKVCache (refuses a freed cache)."""
    desc = getattr(cache, "desc", None)
    if not isinstance(desc, kind) or not desc.reserved:
        raise ValueError("cache is not a live cache made by this library (freed, or another object)")
    return desc


def _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads: int, T: int, B: int, D: int, n_kv_heads: int,
                   head_dim: int) -> None:
    """Dtype, shape and placement of the tensors of a layer call (wq / out may be None for an append)."""
    code = DTYPE_CODES[cache.dtype]
    specs = [(x, "x", dict(code=code, shape=(B, D) if (x.dim() == 2 and T == 1) else (B, T, D)))]
    if wq is not None:
        specs.append((wq, "wq", dict(code=code, shape=(n_q_heads * head_dim, D))))
    specs += [(wk, "wk", dict(code=code, shape=(n_kv_heads * head_dim, D))),
              (wv, "wv", dict(code=code, shape=(n_kv_heads * head_dim, D)))]
    if out is not None:
        specs.append((out, "out", dict(code=code, numel=B * T * n_q_heads * head_dim)))
    if ws is not None:
        specs.append((ws, "ws", {}))
    _tensors(*specs)


def _lens(past_len, batch: int):
    a = np.ascontiguousarray(np.asarray(past_len, dtype=np.int32))
    if a.shape != (batch,):
        raise ValueError(f"past_len must have shape ({batch},), got {a.shape}")
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class HostKVCache:
    """K and V buffers [batch, n_kv_heads, capacity, head_dim] in pinned, mapped host memory
    (hipHostMalloc), read and written in place by the kernels. `k` and `v` are numpy views
    of the same memory (uint16 bit patterns for f16/bf16, float32 for f32)."""

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, capacity: int, dtype: str):
        self.desc = dkv_cache()
        _check(lib().kv_alloc_host(ctypes.byref(self.desc), batch, n_kv_heads, head_dim, capacity,
                                   DTYPE_CODES[dtype]))
        self.dtype = dtype
        self.shape = (batch, n_kv_heads, capacity, head_dim)
        ctype = ctypes.c_float if dtype == "f32" else ctypes.c_uint16
        n = batch * n_kv_heads * capacity * head_dim
        self.k = np.ctypeslib.as_array(ctypes.cast(self.desc.k, ctypes.POINTER(ctype)), shape=(n,)).reshape(self.shape)
        self.v = np.ctypeslib.as_array(ctypes.cast(self.desc.v, ctypes.POINTER(ctype)), shape=(n,)).reshape(self.shape)

    @property
    def batch(self):
        return self.shape[0]

    @property
    def n_kv_heads(self):
        return self.shape[1]

    @property
    def capacity(self):
        return self.shape[2]

    @property
    def head_dim(self):
        return self.shape[3]

    def nbytes(self) -> int:
        return 2 * self.k.nbytes

    def free(self) -> None:
        if self.desc.reserved:
            self.k = self.v = None
            lib().kv_free_host(ctypes.byref(self.desc))

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def kv_append(cache: HostKVCache, x, wk, wv, past_len: Sequence[int], stream=None) -> None:
    """Append round(X·Wkᵀ), round(X·Wvᵀ) at rows [past_len[b], past_len[b]+T). x: [B, T, D]."""
    B, T, D = x.shape
    desc = _cache_desc(cache, dkv_cache)
    _layer_tensors(cache, x, None, wk, wv, None, None, 0, T, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    _check(lib().kv_append(ctypes.byref(desc), _ptr(x), _ptr(wk), _ptr(wv), lp, B, T, D, _stream(stream)))


def workspace_bytes(phase: str, cache: HostKVCache, batch: int, T: int, n_q_heads: int) -> int:
    """Device workspace bytes of a call: "prefill", "decode", or the staging baseline's
    "prefill_staged" / "decode_staged" (which hold a device copy of the whole cache)."""
    ph = {"prefill": 0, "decode": 1, "prefill_staged": 2, "decode_staged": 3}[phase]
    return int(lib().attn_workspace_bytes(ph, ctypes.byref(cache.desc), batch, T, n_q_heads, None))


def attn_prefill(cache: HostKVCache, x, wq, wk, wv, past_len, n_q_heads: int, out, ws, stream=None,
                 rope_theta: float = 0.0) -> None:
    """One prefill step of T tokens per sequence; out: [B, T, Hq*d] device tensor. rope_theta > 0
    rotates q and the new k at positions past_len[b] + t (attn_prefill_rope)."""
    B, T, D = x.shape
    desc = _cache_desc(cache, dkv_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads, T, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    nbytes = ws.numel() * ws.element_size()
    if rope_theta:
        _check(lib().attn_prefill_rope(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, T, D,
                                       n_q_heads, _ptr(out), _ptr(ws), nbytes, float(rope_theta), _stream(stream)))
        return
    _check(lib().attn_prefill(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, T, D,
                              n_q_heads, _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def attn_prefill_variant(cache: HostKVCache, x, wq, wk, wv, past_len, n_q_heads: int, out, ws, variant: str,
                         stream=None) -> None:
    """attn_prefill with the host cache read as `variant` ("fused", "naive", "separate", "staged")."""
    B, T, D = x.shape
    desc = _cache_desc(cache, dkv_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads, T, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().attn_prefill_variant(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, T,
                                      D, n_q_heads, _ptr(out), _ptr(ws), nbytes, _stream(stream),
                                      PREFILL_VARIANTS[variant]))


def attn_decode(cache: HostKVCache, x, wq, wk, wv, past_len, n_q_heads: int, out, ws, stream=None,
                rope_theta: float = 0.0) -> None:
    """One decode step; x: [B, 1, D] (or [B, D]); out: [B, 1, Hq*d] device tensor. rope_theta > 0
    rotates q and the new k at position past_len[b] (attn_decode_rope)."""
    B, D = x.shape[0], x.shape[-1]
    desc = _cache_desc(cache, dkv_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads, 1, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    nbytes = ws.numel() * ws.element_size()
    if rope_theta:
        _check(lib().attn_decode_rope(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, D,
                                      n_q_heads, _ptr(out), _ptr(ws), nbytes, float(rope_theta), _stream(stream)))
        return
    _check(lib().attn_decode(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, D,
                             n_q_heads, _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def attn_decode_noalloc(cache: HostKVCache, x, wq, wk, wv, past_len, n_q_heads: int, out, stream=None) -> None:
    """attn_decode with no workspace: the library's own device scratch (8 MiB per GPU) holds the
    partials, so the call allocates nothing. Calls that may overlap on one GPU must be serialised."""
    B, D = x.shape[0], x.shape[-1]
    desc = _cache_desc(cache, dkv_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, None, n_q_heads, 1, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    _check(lib().attn_decode_noalloc(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, D,
                                     n_q_heads, _ptr(out), _stream(stream)))


class PagedHostKVCache:
    """A pool of 16-token pages in pinned, mapped host memory (hipHostMalloc), read and written
    in place by the kernels, with a free list of physical pages. `k` and `v` are numpy views
    [n_pages, n_kv_heads, 16, head_dim] of the pools (uint16 bit patterns for f16/bf16)."""

    def __init__(self, n_pages: int, n_kv_heads: int, head_dim: int, dtype: str):
        self.desc = dkv_paged_cache()
        _check(lib().kv_paged_alloc_host(ctypes.byref(self.desc), n_pages, n_kv_heads, head_dim, DTYPE_CODES[dtype]))
        self.dtype = dtype
        self.shape = (n_pages, n_kv_heads, PAGE_TOKENS, head_dim)
        ctype = ctypes.c_float if dtype == "f32" else ctypes.c_uint16
        n = n_pages * n_kv_heads * PAGE_TOKENS * head_dim
        self.k = np.ctypeslib.as_array(ctypes.cast(self.desc.k, ctypes.POINTER(ctype)), shape=(n,)).reshape(self.shape)
        self.v = np.ctypeslib.as_array(ctypes.cast(self.desc.v, ctypes.POINTER(ctype)), shape=(n,)).reshape(self.shape)
        self._free = list(range(n_pages - 1, -1, -1))

    @property
    def n_pages(self):
        return self.shape[0]

    @property
    def n_kv_heads(self):
        return self.shape[1]

    @property
    def head_dim(self):
        return self.shape[3]

    def page_bytes(self) -> int:
        """Bytes of one page, K and V."""
        return 2 * self.k[0].nbytes

    def allocate(self, n: int) -> list:
        """Take n free physical pages (raises if the pool is short)."""
        if n > len(self._free):
            raise MemoryError(f"{n} pages requested, {len(self._free)} free")
        return [self._free.pop() for _ in range(n)]

    def release(self, pages) -> None:
        self._free.extend(int(p) for p in pages)

    def memory_stats(self) -> dict:
        """Host bytes of the pool (total and in use); the cache holds no device memory."""
        used = self.n_pages - len(self._free)
        return {"host_bytes_total": self.n_pages * self.page_bytes(), "host_bytes_used": used * self.page_bytes(),
                "device_bytes": 0, "pages_used": used, "pages_free": len(self._free)}

    def free(self) -> None:
        if self.desc.reserved:
            self.k = self.v = None
            lib().kv_paged_free_host(ctypes.byref(self.desc))

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def block_table(page_lists, max_pages: int) -> np.ndarray:
    """int32 [batch, max_pages] block table from per-sequence lists of physical pages (unused
    entries -1)."""
    t = np.full((len(page_lists), max_pages), -1, dtype=np.int32)
    for b, pages in enumerate(page_lists):
        if len(pages) > max_pages:
            raise ValueError(f"sequence {b} maps {len(pages)} pages > max_pages={max_pages}")
        t[b, :len(pages)] = pages
    return t


def _table(table, batch: int):
    t = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
    if t.ndim != 2 or t.shape[0] != batch:
        raise ValueError(f"block table must have shape ({batch}, max_pages), got {t.shape}")
    return t, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), t.shape[1]


def paged_workspace_bytes(phase: str, cache: PagedHostKVCache, batch: int, T: int, n_q_heads: int,
                          max_pages: int) -> int:
    ph = {"prefill": 0, "decode": 1, "append": 2}[phase]
    return int(lib().attn_paged_workspace_bytes(ph, ctypes.byref(cache.desc), batch, T, n_q_heads, max_pages))


def kv_paged_append(cache: PagedHostKVCache, table, x, wk, wv, past_len, ws, stream=None) -> None:
    """kv_append into the pages the block table names. x: [B, T, D]."""
    B, T, D = x.shape
    desc = _cache_desc(cache, dkv_paged_cache)
    _layer_tensors(cache, x, None, wk, wv, None, ws, 0, T, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    t, tp, mp = _table(table, B)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().kv_paged_append(ctypes.byref(desc), tp, mp, _ptr(x), _ptr(wk), _ptr(wv), lp, B, T, D,
                                 _ptr(ws), nbytes, _stream(stream)))


def attn_prefill_paged(cache: PagedHostKVCache, table, x, wq, wk, wv, past_len, n_q_heads: int, out, ws,
                       stream=None) -> None:
    """attn_prefill on a paged cache; out: [B, T, Hq*d] device tensor."""
    B, T, D = x.shape
    desc = _cache_desc(cache, dkv_paged_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads, T, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    t, tp, mp = _table(table, B)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().attn_prefill_paged(ctypes.byref(desc), tp, mp, _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp,
                                    B, T, D, n_q_heads, _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def attn_decode_paged(cache: PagedHostKVCache, table, x, wq, wk, wv, past_len, n_q_heads: int, out, ws,
                      stream=None) -> None:
    """attn_decode on a paged cache; x: [B, 1, D] (or [B, D]); out: [B, 1, Hq*d]."""
    B, D = x.shape[0], x.shape[-1]
    desc = _cache_desc(cache, dkv_paged_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads, 1, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    t, tp, mp = _table(table, B)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().attn_decode_paged(ctypes.byref(desc), tp, mp, _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp,
                                   B, D, n_q_heads, _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def attn_decode_variant(cache: HostKVCache, x, wq, wk, wv, past_len, n_q_heads: int, out, ws, variant: str,
                        stream=None) -> None:
    """attn_decode reading the cache as `variant` ("zerocopy", or "staged": DMA into device memory first)."""
    B, D = x.shape[0], x.shape[-1]
    desc = _cache_desc(cache, dkv_cache)
    _layer_tensors(cache, x, wq, wk, wv, out, ws, n_q_heads, 1, B, D, cache.shape[1], cache.shape[3])
    lens, lp = _lens(past_len, B)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().attn_decode_variant(ctypes.byref(desc), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), lp, B, D,
                                     n_q_heads, _ptr(out), _ptr(ws), nbytes, _stream(stream),
                                     DECODE_VARIANTS[variant]))


def _dtype_code(t) -> int:
    code = _torch_code(t)
    if code is None:
        raise ValueError(f"unsupported dtype {t.dtype} (float32, float16, bfloat16)")
    return code


def rmsnorm(x, weight, y, eps: float = 1e-5, stream=None) -> None:
    """y = x / sqrt(mean(x^2) + eps) * weight over the last axis; y may be x."""
    D = x.shape[-1]
    rows = x.numel() // D
    code = _dtype_code(x)
    _tensors((x, "x", dict(code=code)), (weight, "weight", dict(code=code, shape=(D,))),
             (y, "y", dict(code=code, numel=x.numel())))
    _check(lib().dkv_rmsnorm(_ptr(x), _ptr(weight), _ptr(y), rows, D, eps, code, _stream(stream)))


def linear(x, w, y, residual=None, stream=None) -> None:
    """y = x @ w.T (+ residual); w is a [out, in] weight; residual may be y itself."""
    K = x.shape[-1]
    rows = x.numel() // K
    N = w.shape[0]
    code = _dtype_code(x)
    specs = [(x, "x", dict(code=code)), (w, "w", dict(code=code, shape=(N, K))),
             (y, "y", dict(code=code, numel=rows * N))]
    if residual is not None:
        specs.append((residual, "residual", dict(code=code, numel=rows * N)))
    _tensors(*specs)
    _check(lib().dkv_linear(_ptr(x), _ptr(w), _ptr(residual), _ptr(y), rows, N, K, code, _stream(stream)))


def swiglu(gate_up, y, stream=None) -> None:
    """y = silu(gate) * up for gate_up = [gate, up] on the last axis."""
    F2 = gate_up.shape[-1]
    rows = gate_up.numel() // F2
    code = _dtype_code(gate_up)
    if F2 % 2:
        raise ValueError(f"gate_up's last axis ({F2}) must hold the gate and up halves")
    _tensors((gate_up, "gate_up", dict(code=code)), (y, "y", dict(code=code, numel=rows * (F2 // 2))))
    _check(lib().dkv_swiglu(_ptr(gate_up), _ptr(y), rows, F2 // 2, code, _stream(stream)))


def hostlink_stream(host_ptr: int, nbytes: int, mode: str, n_wg: int = 1024, stream=None) -> None:
    """Kernel streaming read ("read") or write ("write") of pinned host memory."""
    _check(lib().dkv_hostlink_stream(host_ptr, nbytes, {"read": 0, "write": 1}[mode], n_wg, _stream(stream)))


TIMED_PHASES = ("projection", "prefill_attention", "decode_qproj", "decode_attention", "decode_combine")


def timing(enable: bool) -> None:
    """Start (True) or stop (False) recording HIP events around the library's kernel phases;
    either drops what was recorded."""
    _check(lib().dkv_timing(1 if enable else 0))


def timing_read() -> dict:
    """{phase: (milliseconds, launches)} summed over the calls made while timing was on."""
    n = len(TIMED_PHASES)
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib().dkv_timing_read(ms, cnt, n))
    return {name: (float(ms[i]), int(cnt[i])) for i, name in enumerate(TIMED_PHASES)}


def version() -> int:
    return int(lib().dkv_version())
