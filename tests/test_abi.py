"""CPU checks of the C-ABI library: it loads without a GPU and exports every
function that include/zn.h declares (no compute calls are made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zn.h")
LIB = os.path.join(ROOT, "lossless_float_weight_amd", "libzn.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("zn_setup", "zn_setup_transfer", "zn_compress", "zn_decompress"):
        assert required in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libzn.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="libzn.so not built")
def test_status_strings_and_argument_errors_need_no_gpu():
    lib = ctypes.CDLL(LIB)
    lib.zn_status_str.restype = ctypes.c_char_p
    assert lib.zn_status_str(-2) == b"corrupt container"
    # argument checks return before any HIP call
    out = ctypes.c_void_p()
    n = (ctypes.c_uint64 * 1)(1000)
    assert lib.zn_setup(0, None, n, 1, 1000, 0, None, ctypes.byref(out)) == -1   # bad chunk size
    assert lib.zn_setup(7, None, n, 1, 262144, 0, None, ctypes.byref(out)) == -1  # bad dtype
    assert lib.zn_compress(None, None, None, 0, None, None, 0, None) == -1
    assert lib.zn_setup_transfer(None, None, n, 1, None, ctypes.byref(out)) == -1      # no source


@pytest.mark.skipif(not os.path.exists(LIB), reason="libzn.so not built")
def test_kernel_event_names_need_no_gpu():
    lib = ctypes.CDLL(LIB)
    lib.zn_debug_kernel_events.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_void_p]
    for name in (b"analyze", b"finish", b"pack", b"check", b"decode"):
        assert lib.zn_debug_kernel_events(name, None, None) == 0
    assert lib.zn_debug_kernel_events(b"encode", None, None) == -1
    assert lib.zn_debug_kernel_events(None, None, None) == -1


@pytest.mark.skipif(not os.path.exists(LIB), reason="libzn.so not built")
def test_bad_tableset_bytes_and_null_plans_need_no_gpu():
    # a saved plan is parsed and checked before any device memory is taken
    lib = ctypes.CDLL(LIB)
    out = ctypes.c_void_p()
    assert lib.zn_tableset_load(None, 0, ctypes.byref(out)) == -1 and out.value is None
    rng = __import__("random").Random(1)
    for buf in (bytes(64), bytes(rng.randrange(256) for _ in range(4096))):
        b = ctypes.create_string_buffer(buf, len(buf))
        assert lib.zn_tableset_load(b, len(buf), ctypes.byref(out)) == -2     # corrupt
        assert out.value is None
    v = ctypes.c_uint64()
    assert lib.zn_compress_bound(None, ctypes.byref(v)) == -1
    assert lib.zn_scratch_bytes(None, ctypes.byref(v)) == -1
    assert lib.zn_tableset_info(None, None, None, None, None, None, None, None) == -1
    assert lib.zn_decompress(None, None, 0, None, None, 0, 1, None) == -1
