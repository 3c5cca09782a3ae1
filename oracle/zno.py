"""ctypes wrapper of the CPU oracle (liboracle_zno.so).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library and its Python binding
never import this module; the two share no code.

Elements are passed as their raw bit patterns: numpy uint16 for BF16, uint32
for FP32, uint8 for FP8 E4M3 and for FP4 E2M1 pairs (two values per byte).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_zno.so")
SRC = os.path.join(HERE, "zno.c")

BF16, FP32, FP8_E4M3, FP4X2_E2M1 = 0, 1, 2, 3
RAW, CONST, HUFF, GROUP, TANS = 0, 1, 2, 3, 4
CODER_HUFFMAN, CODER_TANS = 0, 1
TANS_LOG = 11
MAX_LEN = 11
ELEM_DTYPE = {BF16: np.uint16, FP32: np.uint32, FP8_E4M3: np.uint8, FP4X2_E2M1: np.uint8}
N_CODED = {BF16: 1, FP32: 4, FP8_E4M3: 2, FP4X2_E2M1: 2}
ALPHABET0 = {BF16: 256, FP32: 256, FP8_E4M3: 16, FP4X2_E2M1: 16}
STATUS = {0: "ok", -1: "argument", -2: "corrupt", -3: "capacity", -4: "tableset", -6: "nomem"}


class OracleError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: oracle status {code} ({STATUS.get(code, '?')})")
        self.code = code


def build(force: bool = True) -> str:
    """Compiles the oracle with gcc (plain C11, no SIMD flags)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                        "-o", tmp, SRC], check=True)
        os.replace(tmp, LIB)
    return LIB


class _Stats(C.Structure):
    _fields_ = [("mode_count", (C.c_uint64 * 5) * 4), ("stream_bytes", C.c_uint64 * 4),
                ("payload_bits", C.c_uint64 * 4), ("raw_plane_bytes", C.c_uint64),
                ("escapes", C.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P, U64, I, U32 = C.c_void_p, C.c_uint64, C.c_int, C.c_uint32
        PU64 = C.POINTER(C.c_uint64)
        L.zno_split.argtypes = [I, P, U64, P, P]
        L.zno_merge.argtypes = [I, P, P, U64, P]
        L.zno_code_lengths.argtypes = [PU64, I, I, P]
        L.zno_group_lengths.argtypes = [PU64, I, I, P]
        L.zno_canonical_codes.argtypes = [P, I, I, P]
        L.zno_compress_bound.argtypes = [I, PU64, I, U32, PU64]
        L.zno_compress.argtypes = [I, C.POINTER(P), PU64, I, U32, P, P, U64, PU64, C.POINTER(_Stats)]
        L.zno_compress2.argtypes = [I, C.POINTER(P), PU64, I, U32, P, I, P, U64, PU64, C.POINTER(_Stats)]
        L.zno_encode_chunk2.argtypes = [I, P, U64, P, I, I, P, U64, PU64, C.POINTER(I)]
        L.zno_tans_normalize.argtypes = [PU64, I, P]
        L.zno_tans_spread.argtypes = [P, I, P]
        L.zno_tans_encode.argtypes = [P, I, P, U64, P, C.POINTER(U32)]
        L.zno_tans_encode.restype = C.c_int64
        L.zno_tans_decode.argtypes = [P, I, P, U64, U32, U64, P]
        L.zno_header.argtypes = [P, U64, C.POINTER(I), C.POINTER(I), PU64, C.POINTER(U32),
                                 C.POINTER(U32), PU64, PU64]
        L.zno_decompress.argtypes = [P, U64, P, C.POINTER(P), PU64, I]
        L.zno_encode_chunk.argtypes = [I, P, U64, P, I, P, U64, PU64, C.POINTER(I)]
        L.zno_setup.argtypes = [I, C.POINTER(P), PU64, I, U32, I, C.POINTER(P)]
        L.zno_setup2.argtypes = [I, C.POINTER(P), PU64, I, U32, I, I, C.POINTER(P)]
        L.zno_tableset_pairs.argtypes = [P, I, C.POINTER(I), C.POINTER(I), P, P]
        L.zno_setup_transfer.argtypes = [P, C.POINTER(P), PU64, I, C.POINTER(P)]
        L.zno_tableset_free.argtypes = [P]
        L.zno_tableset_info.argtypes = [P, C.POINTER(I), C.POINTER(U32), PU64]
        L.zno_tableset_lengths.argtypes = [P, I, P]
        L.zno_tableset_map.argtypes = [P, P]
        L.zno_tableset_cost_history.argtypes = [P, PU64]
        L.zno_tableset_save.argtypes = [P, P, U64, PU64]
        L.zno_tableset_load.argtypes = [P, U64, C.POINTER(P)]
        _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc < 0:
        raise OracleError(rc, where)


def _ptr(a: np.ndarray):
    return C.c_void_p(a.ctypes.data)


def _u64arr(vals):
    a = (C.c_uint64 * len(vals))(*[int(v) for v in vals])
    return a


# ---------------------------------------------------------------- steps ----
def split(dtype: int, x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=ELEM_DTYPE[dtype])
    n = x.size
    planes = np.zeros((N_CODED[dtype], n), np.uint8)
    raw = np.zeros(n, np.uint8)
    lib().zno_split(dtype, _ptr(x), n, _ptr(planes), _ptr(raw))
    return planes, raw


def merge(dtype: int, planes: np.ndarray, raw: np.ndarray) -> np.ndarray:
    planes = np.ascontiguousarray(planes, np.uint8)
    raw = np.ascontiguousarray(raw, np.uint8)
    n = planes.shape[1]
    out = np.zeros(n, ELEM_DTYPE[dtype])
    lib().zno_merge(dtype, _ptr(planes), _ptr(raw), n, _ptr(out))
    return out


def code_lengths(hist, max_len: int = MAX_LEN, group: bool = False) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.uint64))
    out = np.zeros(h.size, np.uint8)
    f = lib().zno_group_lengths if group else lib().zno_code_lengths
    rc = f(h.ctypes.data_as(C.POINTER(C.c_uint64)), h.size, max_len, _ptr(out))
    _check(rc, "code_lengths")
    return out


def canonical_codes(lengths, max_len: int = MAX_LEN) -> np.ndarray:
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    out = np.zeros(ln.size, np.uint32)
    lib().zno_canonical_codes(_ptr(ln), ln.size, max_len, _ptr(out))
    return out


# ----------------------------------------------------------- container ----
def compress_bound(dtype: int, n_elems, chunk_bytes: int) -> int:
    b = C.c_uint64()
    _check(lib().zno_compress_bound(dtype, _u64arr(n_elems), len(n_elems), chunk_bytes,
                                    C.byref(b)), "compress_bound")
    return b.value


def tans_normalize(hist) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.uint64))
    q = np.zeros(h.size, np.uint32)
    _check(lib().zno_tans_normalize(h.ctypes.data_as(C.POINTER(C.c_uint64)), h.size, _ptr(q)), "tans_normalize")
    return q


def tans_spread(q) -> np.ndarray:
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint32))
    out = np.zeros(1 << TANS_LOG, np.uint8)
    lib().zno_tans_spread(_ptr(q), q.size, _ptr(out))
    return out


def tans_encode(q, syms):
    """One segment: (bits as a uint8 array, LSB-first; bit count; final state - 2^11)."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint32))
    x = np.ascontiguousarray(np.asarray(syms, dtype=np.uint8))
    out = np.zeros(2 * x.size + 8, np.uint8)
    st = C.c_uint32()
    nb = lib().zno_tans_encode(_ptr(q), q.size, _ptr(x), x.size, _ptr(out), C.byref(st))
    _check(int(nb) if nb < 0 else 0, "tans_encode")
    return out, int(nb), st.value


def tans_decode(q, bits, nbits: int, state: int, n: int):
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint32))
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8))
    out = np.zeros(max(1, n), np.uint8)
    rc = lib().zno_tans_decode(_ptr(q), q.size, _ptr(b), nbits, state, n, _ptr(out))
    _check(rc, "tans_decode")
    return out[:n]


def compress(dtype: int, tensors, chunk_bytes: int = 262144, ts: "Tableset | None" = None,
             with_stats: bool = False, coder: int = CODER_HUFFMAN):
    """Compresses a list of tensors (bit-pattern arrays) into one container;
    coder selects Huffman or tANS for the exponent stream."""
    if isinstance(tensors, np.ndarray):
        tensors = [tensors]
    arrs = [np.ascontiguousarray(t, dtype=ELEM_DTYPE[dtype]).ravel() for t in tensors]
    n = [a.size for a in arrs]
    cap = compress_bound(dtype, n, chunk_bytes)
    out = np.zeros(cap, np.uint8)
    ptrs = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    nb = C.c_uint64()
    st = _Stats()
    rc = lib().zno_compress2(dtype, ptrs, _u64arr(n), len(arrs), chunk_bytes,
                             ts.handle if ts is not None else None, coder, _ptr(out), cap, C.byref(nb),
                             C.byref(st))
    _check(rc, "compress")
    blob = out[: nb.value].copy()
    if not with_stats:
        return blob
    stats = {
        "mode_count": [[int(st.mode_count[p][m]) for m in range(5)] for p in range(4)],
        "stream_bytes": [int(v) for v in st.stream_bytes],
        "payload_bits": [int(v) for v in st.payload_bits],
        "raw_plane_bytes": int(st.raw_plane_bytes),
        "escapes": int(st.escapes),
    }
    return blob, stats


def header(blob: np.ndarray) -> dict:
    blob = np.ascontiguousarray(blob, np.uint8)
    dt, T = C.c_int(), C.c_int()
    ntot, total, hsh = C.c_uint64(), C.c_uint64(), C.c_uint64()
    cb, nc = C.c_uint32(), C.c_uint32()
    _check(lib().zno_header(_ptr(blob), blob.size, C.byref(dt), C.byref(T), C.byref(ntot),
                            C.byref(cb), C.byref(nc), C.byref(total), C.byref(hsh)), "header")
    return {"dtype": dt.value, "n_tensors": T.value, "n_elems": ntot.value,
            "chunk_bytes": cb.value, "n_chunks": nc.value, "total_bytes": total.value,
            "tableset_hash": hsh.value}


def decompress(blob: np.ndarray, n_elems, dtype: int | None = None, ts: "Tableset | None" = None):
    """Returns the list of decoded tensors; raises OracleError on corrupt input."""
    blob = np.ascontiguousarray(blob, np.uint8)
    if dtype is None:
        dtype = int(blob[6])
    outs = [np.zeros(int(n), ELEM_DTYPE[dtype]) for n in n_elems]
    ptrs = (C.c_void_p * len(outs))(*[o.ctypes.data for o in outs])
    rc = lib().zno_decompress(_ptr(blob), blob.size, ts.handle if ts is not None else None, ptrs,
                              _u64arr(n_elems), len(outs))
    _check(rc, "decompress")
    return outs


def decompress_status(blob: np.ndarray, n_elems, ts: "Tableset | None" = None) -> int:
    """Status code of decoding (for the corruption suite)."""
    blob = np.ascontiguousarray(blob, np.uint8)
    dtype = int(blob[6]) if blob.size > 6 and int(blob[6]) in ELEM_DTYPE else BF16
    outs = [np.zeros(int(n), ELEM_DTYPE[dtype]) for n in n_elems]
    ptrs = (C.c_void_p * len(outs))(*[o.ctypes.data for o in outs])
    return lib().zno_decompress(_ptr(blob), blob.size, ts.handle if ts is not None else None, ptrs,
                                _u64arr(n_elems), len(outs))


def encode_chunk(dtype: int, chunk: np.ndarray, group_len=None, group_id: int = 0,
                 coder: int = CODER_HUFFMAN):
    """Record bytes of one chunk (the container's record for it) and its escape flag."""
    x = np.ascontiguousarray(chunk, ELEM_DTYPE[dtype]).ravel()
    cap = 64 + 4 * (x.size * 4 + 4096)
    rec = np.zeros(cap, np.uint8)
    nb = C.c_uint64()
    esc = C.c_int()
    gl = None
    if group_len is not None:
        gl_arr = np.ascontiguousarray(np.asarray(group_len, np.uint8))
        gl = _ptr(gl_arr)
    _check(lib().zno_encode_chunk2(dtype, _ptr(x), x.size, gl, group_id, coder, _ptr(rec), cap,
                                   C.byref(nb), C.byref(esc)), "encode_chunk")
    return rec[: nb.value].copy(), bool(esc.value)


# ------------------------------------------------------------- tableset ----
class Tableset:
    def __init__(self, handle, dtype: int):
        self.handle = handle
        self.dtype = dtype

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.zno_tableset_free(self.handle)
            self.handle = None

    def info(self):
        K, M, h = C.c_int(), C.c_uint32(), C.c_uint64()
        _check(lib().zno_tableset_info(self.handle, C.byref(K), C.byref(M), C.byref(h)), "info")
        return K.value, M.value, h.value

    @property
    def n_groups(self):
        return self.info()[0]

    @property
    def hash(self):
        return self.info()[2]

    def lengths(self, g: int) -> np.ndarray:
        out = np.zeros(ALPHABET0[self.dtype], np.uint8)
        _check(lib().zno_tableset_lengths(self.handle, g, _ptr(out)), "lengths")
        return out

    def pairs(self, g: int):
        """R9: (packed, F as a list, token lengths[512]) of group g, or None
        when the setup has no pair codes."""
        packed, nf = C.c_int(), C.c_int()
        F = np.zeros(16, np.uint8)
        tl = np.zeros(512, np.uint8)
        rc = lib().zno_tableset_pairs(self.handle, g, C.byref(packed), C.byref(nf), _ptr(F), _ptr(tl))
        _check(rc if rc < 0 else 0, "pairs")
        if rc == 0:
            return None
        return bool(packed.value), F[: nf.value].tolist(), tl

    def group_map(self) -> np.ndarray:
        out = np.zeros(self.info()[1], np.uint8)
        _check(lib().zno_tableset_map(self.handle, _ptr(out)), "map")
        return out

    def cost_history(self) -> np.ndarray:
        out = (C.c_uint64 * 9)()
        _check(lib().zno_tableset_cost_history(self.handle, out), "cost_history")
        return np.array(list(out), np.uint64)

    def save(self) -> bytes:
        n = C.c_uint64()
        _check(lib().zno_tableset_save(self.handle, None, 0, C.byref(n)), "save")
        buf = np.zeros(n.value, np.uint8)
        _check(lib().zno_tableset_save(self.handle, _ptr(buf), n.value, C.byref(n)), "save")
        return buf.tobytes()

    @classmethod
    def load(cls, data: bytes) -> "Tableset":
        buf = np.frombuffer(data, np.uint8).copy()
        h = C.c_void_p()
        _check(lib().zno_tableset_load(_ptr(buf), buf.size, C.byref(h)), "load")
        return cls(h, int(buf[6]))


SETUP_PAIRS = 1


def setup(dtype: int, tensors, chunk_bytes: int = 262144, n_groups: int = 16, pairs: bool = False) -> Tableset:
    if isinstance(tensors, np.ndarray):
        tensors = [tensors]
    arrs = [np.ascontiguousarray(t, ELEM_DTYPE[dtype]).ravel() for t in tensors]
    ptrs = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    h = C.c_void_p()
    _check(lib().zno_setup2(dtype, ptrs, _u64arr([a.size for a in arrs]), len(arrs), chunk_bytes,
                            n_groups, SETUP_PAIRS if pairs else 0, C.byref(h)), "setup")
    return Tableset(h, dtype)


def setup_transfer(src: Tableset, tensors) -> Tableset:
    """The source's group codes for other tensors of its dtype and chunk size,
    each chunk assigned by content to the group code of least coded size."""
    if isinstance(tensors, np.ndarray):
        tensors = [tensors]
    arrs = [np.ascontiguousarray(t, ELEM_DTYPE[src.dtype]).ravel() for t in tensors]
    ptrs = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    h = C.c_void_p()
    _check(lib().zno_setup_transfer(src.handle, ptrs, _u64arr([a.size for a in arrs]), len(arrs),
                                    C.byref(h)), "setup_transfer")
    return Tableset(h, src.dtype)
