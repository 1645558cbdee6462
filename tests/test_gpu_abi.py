"""ABI refusals that need the HIP runtime: a cache descriptor whose k or v is not a pinned host
allocation of the descriptor's size is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _setup():
    import torch
    import zero_copy_host_amd as dkv
    big = dkv.HostKVCache(1, 2, 128, 4096, "bf16")
    small = dkv.HostKVCache(1, 1, 128, 64, "bf16")
    t = dict(x=torch.zeros(1, 1, 256, dtype=torch.bfloat16, device="cuda"),
             wq=torch.zeros(4 * 128, 256, dtype=torch.bfloat16, device="cuda"),
             wk=torch.zeros(2 * 128, 256, dtype=torch.bfloat16, device="cuda"),
             out=torch.zeros(1, 1, 512, dtype=torch.bfloat16, device="cuda"),
             ws=torch.zeros(dkv.workspace_bytes("decode", big, 1, 1, 4), dtype=torch.uint8, device="cuda"))
    return dkv, big, small, t


def _call(dkv, desc, t, past=10):
    import torch
    L = dkv.lib()
    lens = np.array([past], dtype=np.int32)
    lp = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    st = L.attn_decode(ctypes.byref(desc), t["x"].data_ptr(), t["wq"].data_ptr(), t["wk"].data_ptr(),
                       t["wk"].data_ptr(), lp, 1, 256, 4, t["out"].data_ptr(), t["ws"].data_ptr(), t["ws"].numel(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, L.dkv_last_error().decode()


def test_cache_memory_is_checked():
    import torch
    dkv, big, small, t = _setup()
    pageable = np.zeros(2 * 4096 * 128, dtype=np.uint16)
    dev = torch.zeros(2 * 4096 * 128, dtype=torch.bfloat16, device="cuda")
    try:
        assert _call(dkv, big.desc, t)[0] == 0
        d = dkv.dkv_cache.from_buffer_copy(big.desc)
        d.k = dev.data_ptr()
        st, msg = _call(dkv, d, t)
        print("device k:", st, msg)
        assert st == -1 and "not pinned host memory" in msg
        d = dkv.dkv_cache.from_buffer_copy(big.desc)
        d.v = pageable.ctypes.data
        st, msg = _call(dkv, d, t)
        print("pageable v:", st, msg)
        assert st == -1
        # pinned, but too small for the descriptor's shape (another cache's buffer)
        d = dkv.dkv_cache.from_buffer_copy(big.desc)
        d.k = small.desc.k
        st, msg = _call(dkv, d, t)
        print("small pinned k:", st, msg)
        assert st == -1 and "the cache needs" in msg
        # inside its own allocation but shifted by one row: the last row would lie past its end
        d = dkv.dkv_cache.from_buffer_copy(big.desc)
        d.k = big.desc.k + 256
        st, msg = _call(dkv, d, t)
        print("shifted k:", st, msg)
        assert st == -1 and "the cache needs" in msg
        # the same valid call still works afterwards: no error was left behind
        assert _call(dkv, big.desc, t)[0] == 0
    finally:
        big.free()
        small.free()
