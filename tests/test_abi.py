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
    assert lib.zn_compress2(None, 1, None, None, 0, None, None, 0, None) == -1
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


def _header_info(lib, buf: bytes):
    I, U32, U64 = ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64
    P = ctypes.POINTER
    lib.zn_header_info.argtypes = [ctypes.c_void_p, U64, P(I), P(I), P(U64), P(U32), P(U32), P(U64), P(U64)]
    dt, T = I(-1), I(-1)
    n, tot, h = U64(), U64(), U64()
    cb, nc = U32(), U32()
    b = ctypes.create_string_buffer(buf, max(1, len(buf)))
    rc = lib.zn_header_info(b, len(buf), ctypes.byref(dt), ctypes.byref(T), ctypes.byref(n), ctypes.byref(cb),
                            ctypes.byref(nc), ctypes.byref(tot), ctypes.byref(h))
    return rc, {"dtype": dt.value, "n_tensors": T.value, "n_elems": n.value, "chunk_bytes": cb.value,
                "n_chunks": nc.value, "total_bytes": tot.value, "tableset_hash": h.value}


def _oracle_status(oracle, buf: bytes):
    import numpy as np
    try:
        return 0, oracle.header(np.frombuffer(buf, np.uint8))
    except oracle.OracleError as e:
        return e.code, None


@pytest.mark.skipif(not os.path.exists(LIB), reason="libzn.so not built")
def test_header_info_equals_oracle_header_needs_no_gpu(oracle):
    # zn_header_info is host-only; on containers of every dtype (grouped and
    # not) and on every single-byte corruption of their headers it returns
    # the oracle's status and, when it accepts, the oracle's fields
    import numpy as np
    lib = ctypes.CDLL(LIB)
    rng = np.random.default_rng(4)
    blobs = []
    for dt, n in ((oracle.BF16, 70000), (oracle.FP32, 20000), (oracle.FP8_E4M3, 90000),
                  (oracle.FP4X2_E2M1, 50000)):
        x = rng.integers(0, 1 << (8 * oracle.ELEM_DTYPE[dt]().itemsize), n, dtype=np.uint64)
        x = x.astype(oracle.ELEM_DTYPE[dt])
        blobs.append(oracle.compress(dt, [x, x[: n // 3]], 16384))
    g = rng.normal(0, 0.02, 200000).astype(np.float32).view(np.uint32)
    bf = ((g + 0x8000) >> 16).astype(np.uint16)
    ts = oracle.setup(oracle.BF16, [bf], 65536, 2)
    blobs.append(oracle.compress(oracle.BF16, [bf], 65536, ts))
    for blob in blobs:
        hdr = blob[:64].tobytes()
        rc, got = _header_info(lib, hdr)
        orc, want = _oracle_status(oracle, hdr)
        assert rc == orc == 0 and got == want
        for pos in range(64):
            for v in (hdr[pos] ^ 1, hdr[pos] ^ 0x80, 0, 255):
                bad = bytearray(hdr)
                bad[pos] = v
                rc, got = _header_info(lib, bytes(bad))
                orc, want = _oracle_status(oracle, bytes(bad))
                assert rc == orc, (pos, v, rc, orc)
                if rc == 0:
                    assert got == want
    assert _header_info(lib, blobs[0][:63].tobytes())[0] == -1      # too short: argument error
    lib.zn_header_info.argtypes = [ctypes.c_void_p, ctypes.c_uint64] + [ctypes.c_void_p] * 7
    assert lib.zn_header_info(None, 64, *([None] * 7)) == -1


@pytest.mark.skipif(not os.path.exists(LIB), reason="libzn.so not built")
def test_pair_setup_arguments_and_bad_v2_tablesets_need_no_gpu(oracle):
    # zn_setup2's flags are checked before any HIP call; a version-2 saved
    # plan (with packed-pair codes) is validated as the oracle validates it
    import numpy as np
    lib = ctypes.CDLL(LIB)
    out = ctypes.c_void_p()
    n = (ctypes.c_uint64 * 1)(100000)
    I = ctypes.c_int
    lib.zn_setup2.argtypes = [I, ctypes.c_void_p, ctypes.c_void_p, I, ctypes.c_uint32, I, I, ctypes.c_void_p,
                              ctypes.c_void_p]
    assert lib.zn_setup2(1, None, n, 1, 262144, 4, 1, None, ctypes.byref(out)) == -1   # pairs on FP32
    assert lib.zn_setup2(0, None, n, 1, 262144, 0, 1, None, ctypes.byref(out)) == -1   # pairs without groups
    assert lib.zn_setup2(0, None, n, 1, 262144, 4, 2, None, ctypes.byref(out)) == -1   # unknown flag
    rng = np.random.default_rng(1)
    e = 120 + np.minimum(rng.geometric(0.45, 30000), 8)
    e[1::2] = e[0::2]
    x = ((e << 7) | rng.integers(0, 128, e.size)).astype(np.uint16)
    ts = oracle.setup(oracle.BF16, [x], 4096, 2, pairs=True)
    good = ts.save()
    g = next(i for i in range(2) if ts.pairs(i)[0])
    rec = 24 + 8 + 2 * 128 + ts.info()[1] + 274 * g
    muts = [(rec, 2), (rec + 1, 17), (rec + 3, good[rec + 2]), (rec + 18, 0xCC), (rec + 18 + 200, 0x11)]
    for pos, val in muts:
        bad = bytearray(good)
        bad[pos] = val
        try:
            oracle.Tableset.load(bytes(bad))
            want = 0
        except oracle.OracleError as err:
            want = err.code
        b = ctypes.create_string_buffer(bytes(bad), len(bad))
        got = lib.zn_tableset_load(b, len(bad), ctypes.byref(out))
        if want != 0:
            assert got == want == -2, (pos, val, got, want)
