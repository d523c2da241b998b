"""Host-side argument checks of the C ABI: a required tensor pointer that is not
16-byte aligned is refused with RT_EINVAL before anything reaches a device, so
these calls run without a GPU (the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import content_sparse_attention_unit_amd as rt

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "routed_attn.h")


def _enum(name):
    m = re.search(rf"\b{name}\s*=\s*(\d+)", open(HEADER).read())
    assert m, name
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    path = rt.library_path()
    if not os.path.exists(path):
        pytest.skip("library not built")
    h = ctypes.CDLL(path)   # own handle: argtypes set here do not touch the binding's
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    h.rt_route.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                           ctypes.c_size_t, vp]
    h.rt_route.restype = i32
    h.rt_last_error.restype = ctypes.c_char_p
    return h


@pytest.mark.parametrize("bad", ["qk", "mu", "inv_norm", "idx"])
def test_route_rejects_misaligned_pointer(lib, bad):
    ptr = {"qk": 0x10000, "mu": 0x20000, "inv_norm": 0x30000, "idx": 0x40000}
    ptr[bad] += 4   # 4-byte aligned, not 16
    st = lib.rt_route(ptr["qk"], _enum("RT_BF16"), ptr["mu"], 1, 1, 256, 64, 4, 64,
                      ptr["inv_norm"], ptr["idx"], None, None, None, None, 0, None)
    assert st == _enum("RT_EINVAL")
    assert b"16-byte aligned" in lib.rt_last_error()
