"""CPU checks of the C ABI: the library loads, exports every declared
symbol, and its host-side logic (status strings, parameter count, ragged
offsets, argument validation) behaves as documented.  No call here reaches
a device: every invalid call returns before any HIP work."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("lora_pool_create", "lora_segments_build", "lora_bgmv_shrink", "lora_bgmv_expand",
              "lora_sgmv_shrink", "lora_sgmv_expand", "lora_layer_apply"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from lora_bgmv_shrink_amd import binding as b
    lib = b.library()
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(b.EXPORTS) == _declared()


def test_status_strings():
    from lora_bgmv_shrink_amd import binding as b
    lib = b.library()
    for s in range(8):
        assert lib.lora_status_string(s).decode().startswith("LORA_")
    assert b"unknown" in lib.lora_status_string(99)


def test_param_count_closed_form():
    """r(d+k): 131,072 at d=k=4096, r=16 ("Serving many LoRA adapters",
    blog.ecitis.org, "Low-rank structure and additivity")."""
    from lora_bgmv_shrink_amd import binding as b
    assert b.lora_adapter_param_count(16, 4096, 4096) == 131072
    assert b.lora_adapter_param_count(64, 8192, 28672) == 64 * (8192 + 28672)
    assert b.lora_adapter_param_count(0, 4096, 4096) == -1


def test_ragged_offsets():
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl
    ranks = np.array([8, 16, 3, 64, 1, 32], np.int32)
    a_off, b_off, ta, tb = b.lora_pool_ragged_offsets(ranks, 1000, 777)
    # same layout rule as the generator (each block on a 128-element boundary)
    ga, gb, gta, gtb = wl.ragged_layout(ranks, 1000, 777)
    assert a_off.tolist() == ga.tolist() and b_off.tolist() == gb.tolist() and (ta, tb) == (gta, gtb)
    for u in range(len(ranks)):
        assert a_off[u] % 128 == 0 and b_off[u] % 128 == 0
        if u:
            assert a_off[u] >= a_off[u - 1] + 1000 * ranks[u - 1]
            assert b_off[u] >= b_off[u - 1] + ranks[u - 1] * 777
    with pytest.raises(b.LoraError) as e:
        b.lora_pool_ragged_offsets(np.array([8, 65], np.int32), 64, 64)
    assert e.value.status == b.LORA_E_UNSUPPORTED
    with pytest.raises(b.LoraError) as e:
        b.lora_pool_ragged_offsets(np.array([0], np.int32), 64, 64)
    assert e.value.status == b.LORA_E_INVALID


def test_validation_before_any_device_work():
    """Bad arguments are rejected synchronously; null pool / pointers never
    reach a launch."""
    from lora_bgmv_shrink_amd import binding as b
    lib = b.library()
    h = ctypes.c_void_p()
    sc = np.ones(4, np.float32)
    fake = ctypes.c_void_p(0x1000)        # never dereferenced: rejected first
    mis = ctypes.c_void_p(0x1008)         # not 16-byte aligned
    # pool_create
    assert lib.lora_pool_create(None, 0, 1, 4, 64, 64, 16, None, None, None, fake, fake, sc.ctypes.data) == b.LORA_E_INVALID
    assert lib.lora_pool_create(ctypes.byref(h), 0, 7, 4, 64, 64, 16, None, None, None, fake, fake, sc.ctypes.data) == b.LORA_E_INVALID
    assert lib.lora_pool_create(ctypes.byref(h), 0, 1, 0, 64, 64, 16, None, None, None, fake, fake, sc.ctypes.data) == b.LORA_E_INVALID
    assert lib.lora_pool_create(ctypes.byref(h), 0, 1, 4, 64, 64, 65, None, None, None, fake, fake, sc.ctypes.data) == b.LORA_E_UNSUPPORTED
    assert lib.lora_pool_create(ctypes.byref(h), 0, 1, 4, 64, 64, 16, None, None, None, mis, fake, sc.ctypes.data) == b.LORA_E_UNSUPPORTED
    assert lib.lora_pool_create(ctypes.byref(h), 0, 1, 4, 64, 64, 16, None, None, None, None, fake, sc.ctypes.data) == b.LORA_E_INVALID
    # ragged: missing tables, bad rank, overlapping blocks, misaligned offset
    rk = np.array([8, 8], np.int32)
    ao = np.array([0, 64 * 8], np.int64)
    bo = np.array([0, 8 * 64], np.int64)
    sc2 = np.ones(2, np.float32)
    assert lib.lora_pool_create(ctypes.byref(h), 1, 1, 2, 64, 64, 8, None, ao.ctypes.data, bo.ctypes.data, fake, fake, sc2.ctypes.data) == b.LORA_E_INVALID
    bad_rk = np.array([8, 9], np.int32)
    assert lib.lora_pool_create(ctypes.byref(h), 1, 1, 2, 64, 64, 8, bad_rk.ctypes.data, ao.ctypes.data, bo.ctypes.data, fake, fake, sc2.ctypes.data) == b.LORA_E_INVALID
    ov = np.array([0, 64 * 8 - 8], np.int64)
    assert lib.lora_pool_create(ctypes.byref(h), 1, 1, 2, 64, 64, 8, rk.ctypes.data, ov.ctypes.data, bo.ctypes.data, fake, fake, sc2.ctypes.data) == b.LORA_E_INVALID
    odd = np.array([0, 64 * 8 + 3], np.int64)
    assert lib.lora_pool_create(ctypes.byref(h), 1, 1, 2, 64, 64, 8, rk.ctypes.data, odd.ctypes.data, bo.ctypes.data, fake, fake, sc2.ctypes.data) == b.LORA_E_UNSUPPORTED
    # hot calls with a null pool
    assert lib.lora_bgmv_shrink(None, fake, 64, fake, 4, fake, 16, None) == b.LORA_E_INVALID
    assert lib.lora_bgmv_expand(None, fake, 16, fake, 4, fake, 1, 64, 0, None) == b.LORA_E_INVALID
    assert lib.lora_sgmv_shrink(None, fake, 64, None, 4, fake, 16, None, 0, None) == b.LORA_E_INVALID
    assert lib.lora_sgmv_expand(None, fake, 16, None, 4, fake, 1, 64, 0, None) == b.LORA_E_INVALID
    assert lib.lora_layer_apply(None, fake, 64, fake, 64, 0, fake, None, 4, fake, 1, 64, 0, None, 0, None) == b.LORA_E_INVALID
    # segments: bad sizes, missing descriptor, too-small capacity, too many adapters
    seg = b.SegmentsT(0x1000, 0x1000, 0x1000, 0x1000, 2)
    assert lib.lora_segments_build(fake, 10, 0, ctypes.byref(seg), None, None, 0, None) == b.LORA_E_INVALID
    assert lib.lora_segments_build(fake, 10, 4, None, None, None, 0, None) == b.LORA_E_INVALID
    assert lib.lora_segments_build(fake, 10, 4, ctypes.byref(seg), None, None, 0, None) == b.LORA_E_INVALID
    big = b.SegmentsT(0x1000, 0x1000, 0x1000, 0x1000, 100000)
    assert lib.lora_segments_build(fake, 10, 20000, ctypes.byref(big), None, None, 0, None) == b.LORA_E_UNSUPPORTED
    ws = ctypes.c_size_t(123)
    assert lib.lora_segments_workspace(10, 4, ctypes.byref(ws)) == b.LORA_OK and ws.value == 0
    assert lib.lora_workspace_clear(mis, 64, None) == b.LORA_E_INVALID
    assert lib.lora_workspace_clear(None, 0, None) == b.LORA_OK


def test_product_path_does_not_import_oracle():
    """The binding and the kernels never reach the oracle."""
    pkg = os.path.join(ROOT, "lora_bgmv_shrink_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "lora_oracle" not in text, f
