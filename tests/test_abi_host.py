"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host with the documented codes
before touching the device."""

import ctypes
import os
import re

import pytest

from block_sparse_long_bsattn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b((?:bsattn|lfattn)_\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_exports():
    names = declared_functions()
    assert len(names) == 25, names
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert _lib.bsattn_status_str(0) == "BSATTN_OK"
    assert _lib.bsattn_status_str(-1) == "BSATTN_EINVAL"
    assert _lib.bsattn_status_str(-2) == "BSATTN_EUNSUPPORTED"
    assert _lib.bsattn_status_str(-3) == "BSATTN_EHIP"
    assert _lib.bsattn_status_str(-4) == "BSATTN_ENOMEM"
    assert "gfx950" in _lib.bsattn_version()


def _build_status(n, b, heads, G, w, r):
    lib = _lib.load()
    arr = (ctypes.c_int32 * max(1, len(G)))(*G)
    out = ctypes.c_void_p(12345)
    st = lib.bsattn_layout_build(n, b, heads, arr if G else None, len(G), w, r, 1, None,
                                 ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("args,code", [
    ((0, 64, 1, [], 3, 3), -1),             # empty sequence
    ((500, 64, 1, [8], 3, 3), -1),          # block 8 past ceil(500/64) = 8 blocks
    ((512, 32, 1, [0], 3, 3), -2),          # block size other than 64
    ((512, 64, 0, [0], 3, 3), -1),          # no heads
    ((512, 64, 1, [0], 2, 3), -1),          # even window
    ((512, 64, 1, [0], 0, 3), -1),          # empty window
    ((512, 64, 1, [0], 3, -1), -1),         # negative r
    ((512, 64, 1, [0], 3, 65), -2),         # r above the built limit
    ((512, 64, 1, [7, 0], 3, 3), -1),       # unsorted global set
    ((512, 64, 1, [3, 3], 3, 3), -1),       # duplicate
    ((512, 64, 1, [8], 3, 3), -1),          # out of range
    ((64 * 4097, 64, 1, [0], 3, 3), -2),    # too many blocks
])
def test_layout_build_rejects_bad_arguments(args, code):
    st, out = _build_status(*args)
    assert st == code
    assert out is None                      # *out cleared on failure
    assert _lib.bsattn_last_error() != ""


def test_null_handles_are_rejected():
    lib = _lib.load()
    assert lib.bsattn_fwd(None, 1, 64, 1, 0.125, *([None] * 6), None, 0, None) == -1
    assert lib.bsattn_bwd(None, 1, 64, 1, 0.125, *([None] * 10), None, 0, None) == -1
    assert lib.bsattn_bwd_noalloc(None, 1, 64, 1, 0.125, *([None] * 10), None) == -1
    assert lib.lfattn_fwd(None, 1, 1, 64, 1, 0.125, *([None] * 6), None, 0, None) == -1
    assert lib.lfattn_bwd(None, 1, 1, 64, 1, 0.125, *([None] * 10), None, 0, None) == -1
    assert lib.lfattn_fwd_gproj(None, 1, 1, 64, 1, 0.125, *([None] * 9), None, 0, None) == -1
    assert lib.lfattn_bwd_gproj(None, 1, 1, 64, 1, 0.125, *([None] * 16), None, 0, None) == -1
    assert lib.bsattn_layout_info(None, None, None, None) == -1
    assert lib.bsattn_layout_rebuild(None, 1, None) == -1
    assert lib.bsattn_fwd_workspace(None, 1, 64) == 0
    assert lib.bsattn_bwd_workspace(None, 1, 64) == 0
    assert lib.lfattn_fwd_workspace(None, 1, 1, 64) == 0
    assert lib.lfattn_bwd_workspace(None, 1, 1, 64) == 0
    assert lib.lfattn_plan_build_dilated(100, 1, None, 0, 1, None, 0, None, None) == -1
    assert lib.bsattn_layout_destroy(None) == 0
    assert lib.lfattn_plan_destroy(None) == 0
    assert lib.bsattn_profile_read(-1, None, None, None, None) == -1


@pytest.mark.parametrize("args,code", [
    ((0, 16, [], 0), -1),          # empty sequence
    ((512, -1, [0], 1), -1),       # negative window
    ((512, 16, [5, 1], 2), -1),    # unsorted
    ((512, 16, [512], 1), -1),     # out of range
    ((64 * 4097, 16, [0], 1), -2), # longer than the built limit
])
def test_lf_plan_rejects_bad_arguments(args, code):
    lib = _lib.load()
    n, w1, G, ng = args
    arr = (ctypes.c_int32 * len(G))(*G)
    out = ctypes.c_void_p(7)
    assert lib.lfattn_plan_build(n, w1, arr, ng, None, ctypes.byref(out)) == code
    assert out.value is None


def test_missing_library_fails_loudly(tmp_path):
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(RuntimeError, match="no fallback"):
            _lib.load(str(tmp_path / "nope.so"))
    finally:
        _lib._lib = saved


@pytest.mark.parametrize("args,code", [
    ((512, 8, [0], 2, [0, 1], 1), -1),      # causal window with a global token
    ((512, 8, [], 2, [0, -1], 0), -1),      # negative dilation
    ((512, 8, [], 2, [0, 1024], 0), -1),    # dilation above the limit
    ((512, 8, [], 0, [], 0), -1),           # no heads
    ((512, 8, [], 4097, None, 0), -1),      # too many heads
    ((512, 8, [], 1, [0], 2), -1),          # causal flag not 0/1
    ((0, 8, [], 1, [0], 0), -1),            # empty sequence
    ((512, 1 << 21, [], 1, [1023], 0), -2), # window span above 2^30
])
def test_dilated_plan_rejects_bad_arguments(args, code):
    lib = _lib.load()
    n, w1, G, heads, dil, causal = args
    garr = (ctypes.c_int32 * max(1, len(G)))(*G)
    darr = None if dil is None else (ctypes.c_int32 * len(dil))(*dil)
    out = ctypes.c_void_p(7)
    st = lib.lfattn_plan_build_dilated(n, w1, garr if G else None, len(G), heads, darr, causal,
                                       None, ctypes.byref(out))
    assert st == code
    assert out.value is None
    assert _lib.bsattn_last_error() != ""


@pytest.mark.parametrize("args,code", [
    ((-1, 100, 8, 3), -1),       # negative g
    ((4, 0, 8, 3), -1),          # no ordinary tokens
    ((4, 100, 0, 3), -1),        # empty blocks
    ((4, 100, 8, 2), -1),        # even window
    ((4, 100, 8, -1), -1),       # negative window
    ((200000, 62145, 84, 3), -2),  # g + n above the limit
])
def test_etc_plan_rejects_bad_arguments(args, code):
    lib = _lib.load()
    out = ctypes.c_void_p(7)
    assert lib.lfattn_plan_build_etc(*args, None, ctypes.byref(out)) == code
    assert out.value is None
    assert _lib.bsattn_last_error() != ""
