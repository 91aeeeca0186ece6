"""The C-ABI library loads and exports every entry point include/*.h declares.

No compute calls (no GPU here): loading libhisparse.so only needs the HIP
runtime library, and the host-side argument checks that touch no device
state can run too.
"""
import ctypes
import glob
import os
import re

import pytest

from tiered_kv_cache_hs_amd import hisparse as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(hs_[a-z_0-9]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_header_declares_the_binding_names():
    assert declared_functions() == set(H.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = H.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings_and_tuning_roundtrip():
    assert H.hs_status_str(H.HS_OK) == "ok"
    assert H.hs_status_str(H.HS_E_STATE) == "invalid buffer state"
    assert H.hs_status_str(H.HS_E_DEVICE) == "data error reported by the device"
    assert (H.HS_E_DEVICE, H.HS_E_STATE) == (-5, -6)
    H.hs_set_tuning(4, 96, 2, 64, 32, 2)
    assert H.hs_get_tuning() == {"attn_splits": 4, "latent_heads_per_wg": 32,
                                 "prefetch_workgroups": 96, "prefetch_batch": 2,
                                 "gather_bytes_per_lane": 64, "resolve_fetch": 2}
    H.hs_set_tuning()
    for gb in (16, 32, 128):
        H.hs_set_tuning(gather_bytes_per_lane=gb)
        assert H.hs_get_tuning()["gather_bytes_per_lane"] == gb
    for gb in (8, 48, 256, -16):
        with pytest.raises(H.HsError):
            H.hs_set_tuning(gather_bytes_per_lane=gb)
    H.hs_set_tuning()
    with pytest.raises(H.HsError):
        H.hs_set_tuning(-1)
    with pytest.raises(H.HsError):
        H.hs_set_tuning(prefetch_workgroups=-3)
    with pytest.raises(H.HsError):
        H.hs_set_tuning(prefetch_batch=3)
    for hpw in (16, 48, -32):
        with pytest.raises(H.HsError):
            H.hs_set_tuning(latent_heads_per_wg=hpw)
    for rf in (-1, 3):
        with pytest.raises(H.HsError):
            H.hs_set_tuning(resolve_fetch=rf)
    assert H.hs_get_tuning()["prefetch_workgroups"] == 0


def test_null_and_shape_checks_without_device():
    L = H.lib()
    assert L.hs_pool_create(None, None) == H.HS_E_INVAL
    assert L.hs_batch_create(None, 0, None) == H.HS_E_INVAL
    assert L.hs_resolve(None, None, 1, None, None, None) == H.HS_E_INVAL
    # descriptor checks that come before any allocation
    d = H.PoolDesc(1, 1, H.HS_KV_MHA, H.HS_F32, 1, 8, 0, 0, (ctypes.c_int64 * 1)(100), None, 48)
    assert L.hs_pool_create(ctypes.byref(d), ctypes.byref(ctypes.c_void_p())) == H.HS_E_INVAL
    d = H.PoolDesc(1, 1, H.HS_KV_MHA, H.HS_F32, 1, 8, 0, 0, (ctypes.c_int64 * 1)(100),
                   (ctypes.c_int64 * 1)(99), 0)  # maximum below the capacity
    assert L.hs_pool_create(ctypes.byref(d), ctypes.byref(ctypes.c_void_p())) == H.HS_E_INVAL
    assert L.hs_pool_reserve(None, 0, 10) == H.HS_E_INVAL
    assert L.hs_pool_record_ptr(None, 0, 0, 0, None, None) == H.HS_E_INVAL
    assert L.hs_buffer_bytes(None, 4) == 0
    assert L.hs_buffer_shared_bytes(None, 4) == 0
    assert L.hs_buffer_create_shared(None, 0, None, 0, None) == H.HS_E_INVAL
    assert L.hs_buffer_grow_group(None, None, 0, 4, None, 0, None, None, None) == H.HS_E_INVAL
    assert L.hs_prefetch(None, None) == H.HS_E_INVAL
    assert L.hs_pool_append_batch(None, None, None) == H.HS_E_INVAL
    assert L.hs_batch_status(None, None, None) == H.HS_E_INVAL
    assert L.hs_stage_create(None, 0, 1, None) == H.HS_E_INVAL
    assert L.hs_stage_run(None, None) == H.HS_E_INVAL
    assert L.hs_stage_set_step(None, 0, None) == H.HS_E_INVAL
    assert L.hs_stage_get_step(None, None) == H.HS_E_INVAL
    assert L.hs_stage_destroy(None) == H.HS_E_INVAL
    # stage regions are checked before anything is allocated
    st = ctypes.c_void_p()
    bad = [H.StageRegion(0x1000, 0x9000, 24, 32)]  # 24 bytes: not a multiple of 16
    assert L.hs_stage_create((H.StageRegion * 1)(*bad), 1, 4, ctypes.byref(st)) == H.HS_E_INVAL
    assert "multiples of 16" in H.hs_last_error()
    bad = [H.StageRegion(0x1000, 0x1020, 32, 32)]  # destination inside the source ring
    assert L.hs_stage_create((H.StageRegion * 1)(*bad), 1, 4, ctypes.byref(st)) == H.HS_E_INVAL
    bad = [H.StageRegion(0x1000, 0x9000, 32, 32), H.StageRegion(0x5000, 0x9010, 32, 32)]
    assert L.hs_stage_create((H.StageRegion * 2)(*bad), 2, 4, ctypes.byref(st)) == H.HS_E_INVAL
    assert "overlaps" in H.hs_last_error()
    many = [H.StageRegion(0x1000 * (i + 1), 0x100000 + 0x1000 * i, 32, 32) for i in range(9)]
    assert L.hs_stage_create((H.StageRegion * 9)(*many), 9, 1, ctypes.byref(st)) == H.HS_E_INVAL
    assert "1 to 8 regions" in H.hs_last_error()
    d = H.PoolDesc(1, 1, 7, H.HS_BF16, 1, 64, 0, 0, (ctypes.c_int64 * 1)(100))
    out = ctypes.c_void_p()
    assert L.hs_pool_create(ctypes.byref(d), ctypes.byref(out)) == H.HS_E_INVAL
    d = H.PoolDesc(1, 1, H.HS_KV_MHA, H.HS_BF16, 1, 3, 0, 0, (ctypes.c_int64 * 1)(100))
    assert L.hs_pool_create(ctypes.byref(d), ctypes.byref(out)) == H.HS_E_INVAL  # 12-byte record
    assert "multiple of 16" in H.hs_last_error()
