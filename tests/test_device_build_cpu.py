"""The device layout build's host-side contract (no device work): workspace sizing and the
argument errors returned before anything reaches the GPU."""
import ctypes

import numpy as np

from ad_recommendation_amd import emb


def test_workspace_grows_with_keys_and_covers_the_buffers():
    a = emb.table_build_workspace_bytes([16], 1, 0.5, 1000)
    b = emb.table_build_workspace_bytes([16], 1, 0.5, 1_000_000)
    c = emb.table_build_workspace_bytes([16], 2, 0.5, 1_000_000)
    assert 0 < a < b <= c
    # keys (8 B), four sort buffers (16 B) and buckets for 2N home slots plus overflow (>= 17 B)
    assert b >= 1_000_000 * (8 + 16 + 17)
    assert emb.table_build_workspace_bytes([16], 1, 0.5, 0) > 0


def test_errors_before_any_device_work():
    L = emb.lib()
    dims = (ctypes.c_int32 * 1)(16)
    desc = emb.EmbTableDesc(1, dims, 0, 0, 1, 0.5, 0.1, 0)
    keys = np.arange(1, 11, dtype=np.int64)
    h = ctypes.c_void_p()
    n = ctypes.c_size_t()
    assert L.table_build_workspace_bytes(ctypes.byref(desc), 1 << 31, ctypes.byref(n)) == -4
    assert L.table_build_workspace_bytes(ctypes.byref(desc), -1, ctypes.byref(n)) == -4
    bad = emb.EmbTableDesc(1, dims, 0, 0, 1, 0.0, 0.1, 0)
    assert L.table_build_workspace_bytes(ctypes.byref(bad), 10, ctypes.byref(n)) == -1
    kp = keys.ctypes.data
    assert L.table_create_on_device(ctypes.byref(desc), kp, 10, None, 1 << 20, None, ctypes.byref(h)) == -1
    assert L.table_create_on_device(ctypes.byref(desc), kp, 10, 4096 + 16, 1 << 20, None, ctypes.byref(h)) == -1
    assert L.table_create_on_device(ctypes.byref(desc), kp, 1 << 31, 4096, 1 << 40, None, ctypes.byref(h)) == -4
    # descriptor errors come before the device: a bad dim
    d12 = (ctypes.c_int32 * 1)(12)
    desc12 = emb.EmbTableDesc(1, d12, 0, 0, 1, 0.5, 0.1, 0)
    assert L.table_create_on_device(ctypes.byref(desc12), kp, 10, 4096, 1 << 20, None, ctypes.byref(h)) == -1
