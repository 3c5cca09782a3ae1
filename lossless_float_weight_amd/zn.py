"""Python binding of libzn.so (include/zn.h): argument marshalling only.

Every step of setup, compression and decompression runs in the library's HIP
kernels; this module turns torch tensors into device pointers and streams,
and raises ZnError on a non-zero status.  There is no fallback: if libzn.so
is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzn.so")

BF16, FP32, FP8_E4M3, FP4X2_E2M1 = 0, 1, 2, 3
CODER_HUFFMAN, CODER_TANS = 0, 1
SETUP_PAIRS = 1
# FP4 E2M1 pairs travel as uint8 tensors (two values per byte, low nibble first)
TORCH_DTYPE = {BF16: torch.bfloat16, FP32: torch.float32, FP8_E4M3: torch.float8_e4m3fn,
               FP4X2_E2M1: torch.uint8}
ZN_DTYPE = {v: k for k, v in TORCH_DTYPE.items()}
STATUS = {0: "ok", -1: "invalid argument", -2: "corrupt container", -3: "buffer too small",
          -4: "tableset mismatch", -5: "HIP runtime error", -6: "out of memory"}
ROUNDS = 8


class ZnError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, 'status %d' % code)}")
        self.code = code


_lib = None


def lib() -> C.CDLL:
    """Loads libzn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ZnError(-1, f"libzn.so not built at {LIB_PATH} (run python lossless_float_weight_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        P, U64, I, U32 = C.c_void_p, C.c_uint64, C.c_int, C.c_uint32
        PU64 = C.POINTER(C.c_uint64)
        L.zn_setup.argtypes = [I, C.POINTER(P), PU64, I, U32, I, P, C.POINTER(P)]
        L.zn_setup2.argtypes = [I, C.POINTER(P), PU64, I, U32, I, I, P, C.POINTER(P)]
        L.zn_tableset_pairs.argtypes = [P, I, C.POINTER(I), C.POINTER(I), C.POINTER(I), P, P]
        L.zn_setup_transfer.argtypes = [P, C.POINTER(P), PU64, I, P, C.POINTER(P)]
        L.zn_plan_from_container.argtypes = [P, U64, P, C.POINTER(P)]
        L.zn_header_info.argtypes = [P, U64, C.POINTER(I), C.POINTER(I), PU64, C.POINTER(U32),
                                     C.POINTER(U32), PU64, PU64]
        L.zn_tableset_info.argtypes = [P, C.POINTER(I), C.POINTER(I), PU64, C.POINTER(U32),
                                       C.POINTER(U32), C.POINTER(I), PU64]
        L.zn_compress_bound.argtypes = [P, PU64]
        L.zn_scratch_bytes.argtypes = [P, PU64]
        L.zn_compress.argtypes = [P, P, P, U64, PU64, P, U64, P]
        L.zn_compress2.argtypes = [P, I, P, P, U64, PU64, P, U64, P]
        L.zn_decompress.argtypes = [P, P, U64, P, P, U64, I, P]
        L.zn_decompress_noalloc.argtypes = [P, P, U64, P, P, I, P]
        L.zn_tableset_save.argtypes = [P, P, U64, PU64]
        L.zn_tableset_load.argtypes = [P, U64, C.POINTER(P)]
        L.zn_tableset_lengths.argtypes = [P, I, P]
        L.zn_tableset_map.argtypes = [P, P]
        L.zn_tableset_cost_history.argtypes = [P, PU64]
        L.zn_tableset_free.argtypes = [P]
        L.zn_status_str.restype = C.c_char_p
        L.zn_debug_histograms.argtypes = [P, P, P, P]
        L.zn_debug_code_lengths.argtypes = [P, I, I, I, P, P]
        L.zn_debug_kernel_events.argtypes = [C.c_char_p, P, P]
        for f in ("zn_setup", "zn_setup_transfer", "zn_plan_from_container", "zn_header_info",
                  "zn_tableset_info", "zn_compress_bound",
                  "zn_scratch_bytes", "zn_compress", "zn_decompress", "zn_decompress_noalloc",
                  "zn_tableset_save",
                  "zn_tableset_load", "zn_tableset_lengths", "zn_tableset_map",
                  "zn_tableset_cost_history", "zn_debug_histograms", "zn_debug_code_lengths",
                  "zn_debug_kernel_events"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise ZnError(rc, where)


def _stream(stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr_array(tensors: Sequence[torch.Tensor], device, stream=None) -> torch.Tensor:
    """Device array of the tensors' data pointers (the ABI's d_*_ptrs), its
    copy ordered on the stream the call runs on."""
    vals = torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64)
    if stream is None:
        return vals.to(device)
    with torch.cuda.stream(stream):
        return vals.to(device)


def _u64(vals):
    return (C.c_uint64 * len(vals))(*[int(v) for v in vals])


class Tableset:
    """Owns a zn_tableset handle (the plan and optional group tables)."""

    def __init__(self, handle: C.c_void_p):
        self.handle = handle

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.zn_tableset_free(h)
            self.handle = None

    def info(self) -> dict:
        """Plan facts (fixed for the handle's lifetime, so read once)."""
        if getattr(self, "_info", None) is None:
            self._info = self._read_info()
        return dict(self._info)

    def _read_info(self) -> dict:
        dt, T, nc, K = C.c_int(), C.c_int(), C.c_uint32(), C.c_int()
        cb, h = C.c_uint32(), C.c_uint64()
        _check(lib().zn_tableset_info(self.handle, C.byref(dt), C.byref(T), None, C.byref(cb),
                                      C.byref(nc), C.byref(K), C.byref(h)), "tableset_info")
        n = (C.c_uint64 * T.value)()
        _check(lib().zn_tableset_info(self.handle, None, None, n, None, None, None, None),
               "tableset_info")
        return {"dtype": dt.value, "n_tensors": T.value, "n_elems": [int(v) for v in n],
                "chunk_bytes": cb.value, "n_chunks": nc.value, "n_groups": K.value,
                "hash": h.value}

    @property
    def dtype(self) -> int:
        return self.info()["dtype"]

    @property
    def n_groups(self) -> int:
        return self.info()["n_groups"]

    @property
    def hash(self) -> int:
        return self.info()["hash"]

    def lengths(self, g: int) -> list:
        A = 16 if self.dtype in (FP8_E4M3, FP4X2_E2M1) else 256
        buf = (C.c_uint8 * A)()
        _check(lib().zn_tableset_lengths(self.handle, g, buf), "tableset_lengths")
        return list(buf)

    def pairs(self, g: int):
        """Group g's packed-pair code: (packs, F as a list, token lengths as a
        list of 512), or None when the setup has no pair codes."""
        has, packed, nf = C.c_int(), C.c_int(), C.c_int()
        F = (C.c_uint8 * 16)()
        tl = (C.c_uint8 * 512)()
        _check(lib().zn_tableset_pairs(self.handle, g, C.byref(has), C.byref(packed), C.byref(nf), F, tl),
               "tableset_pairs")
        if not has.value:
            return None
        return bool(packed.value), list(F)[: nf.value], list(tl)

    def group_map(self) -> list:
        buf = (C.c_uint8 * max(1, self.info()["n_chunks"]))()
        _check(lib().zn_tableset_map(self.handle, buf), "tableset_map")
        return list(buf)[: self.info()["n_chunks"]]

    def cost_history(self) -> list:
        buf = (C.c_uint64 * (ROUNDS + 1))()
        _check(lib().zn_tableset_cost_history(self.handle, buf), "cost_history")
        return [int(v) for v in buf]

    def save(self) -> bytes:
        n = C.c_uint64()
        _check(lib().zn_tableset_save(self.handle, None, 0, C.byref(n)), "tableset_save")
        buf = (C.c_uint8 * n.value)()
        _check(lib().zn_tableset_save(self.handle, buf, n.value, C.byref(n)), "tableset_save")
        return bytes(buf)

    @classmethod
    def load(cls, data: bytes) -> "Tableset":
        buf = (C.c_uint8 * len(data)).from_buffer_copy(data)
        h = C.c_void_p()
        _check(lib().zn_tableset_load(buf, len(data), C.byref(h)), "tableset_load")
        return cls(h)


def setup(tensors: Sequence[torch.Tensor] | None = None, *, dtype=None, n_elems=None,
          chunk_bytes: int = 262144, n_groups: int = 0, pairs: bool = False, stream=None) -> Tableset:
    """zn_setup (zn_setup2 with pairs): a plan for these tensor sizes; with
    n_groups > 0 the chunks of `tensors` are grouped and share code tables;
    pairs adds packed exponent pairs (BF16)."""
    if tensors is not None:
        tensors = [t.contiguous() for t in tensors]
        dtype = ZN_DTYPE[tensors[0].dtype]
        n_elems = [t.numel() for t in tensors]
        ptrs = (C.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    else:
        ptrs = None
        dtype = ZN_DTYPE.get(dtype, dtype)
    h = C.c_void_p()
    # the tableset lives on the tensors' device (else on the current one)
    with torch.cuda.device(tensors[0].device if tensors else None):
        _check(lib().zn_setup2(int(dtype), ptrs, _u64(n_elems), len(n_elems), chunk_bytes, n_groups,
                               SETUP_PAIRS if pairs else 0, _stream(stream), C.byref(h)), "setup")
    return Tableset(h)


def setup_transfer(src: Tableset, tensors: Sequence[torch.Tensor], stream=None) -> Tableset:
    """zn_setup_transfer: src's group codes for these tensors (same dtype and
    chunk size), each chunk assigned by content to its cheapest group code."""
    want = TORCH_DTYPE[src.info()["dtype"]]
    if any(t.dtype != want for t in tensors):
        raise ZnError(-1, f"setup_transfer: the source tableset codes {want}, got "
                          f"{sorted(set(str(t.dtype) for t in tensors))}")
    tensors = [t.contiguous() for t in tensors]
    ptrs = (C.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    h = C.c_void_p()
    with torch.cuda.device(tensors[0].device):
        _check(lib().zn_setup_transfer(src.handle, ptrs, _u64([t.numel() for t in tensors]), len(tensors),
                                       _stream(stream), C.byref(h)), "setup_transfer")
    return Tableset(h)


def plan_from_container(blob: torch.Tensor, stream=None) -> Tableset:
    h = C.c_void_p()
    with torch.cuda.device(blob.device):
        _check(lib().zn_plan_from_container(C.c_void_p(blob.data_ptr()), blob.numel(), _stream(stream),
                                            C.byref(h)), "plan_from_container")
    return Tableset(h)


def header_info(hdr) -> dict:
    """zn_header_info on the first 64 bytes of a container (host bytes, a
    numpy array or a tensor on any device)."""
    if isinstance(hdr, torch.Tensor):
        hdr = hdr[:64].cpu().numpy().tobytes()
    elif not isinstance(hdr, (bytes, bytearray)):
        hdr = bytes(memoryview(hdr)[:64])
    buf = (C.c_uint8 * max(1, len(hdr))).from_buffer_copy(bytes(hdr) or b"\0")
    dt, T = C.c_int(), C.c_int()
    n, tot, h = C.c_uint64(), C.c_uint64(), C.c_uint64()
    cb, nc = C.c_uint32(), C.c_uint32()
    _check(lib().zn_header_info(buf, len(hdr), C.byref(dt), C.byref(T), C.byref(n), C.byref(cb),
                                C.byref(nc), C.byref(tot), C.byref(h)), "header_info")
    return {"dtype": dt.value, "n_tensors": T.value, "n_elems": n.value, "chunk_bytes": cb.value,
            "n_chunks": nc.value, "total_bytes": tot.value, "tableset_hash": h.value}


def _check_tensors(ts: Tableset, tensors, where: str, exact: bool) -> None:
    """The tensors must be the plan's: count, dtype, one CUDA device,
    contiguous storage, and exactly (inputs) or at least (outputs) the
    plan's element counts.  Raises ZnError(-1) before any launch."""
    info = ts.info()
    want = TORCH_DTYPE[info["dtype"]]
    if len(tensors) != info["n_tensors"]:
        raise ZnError(-1, f"{where}: plan has {info['n_tensors']} tensors, got {len(tensors)}")
    dev = None
    for i, (t, n) in enumerate(zip(tensors, info["n_elems"])):
        if t.dtype != want:
            raise ZnError(-1, f"{where}: tensor {i} is {t.dtype}, the plan codes {want}")
        if not t.is_cuda or (dev is not None and t.device != dev):
            raise ZnError(-1, f"{where}: tensor {i} is not on the plan's CUDA device")
        dev = t.device
        if not t.is_contiguous():
            raise ZnError(-1, f"{where}: tensor {i} is not contiguous (pass .contiguous())")
        if (t.numel() != n) if exact else (t.numel() < n):
            raise ZnError(-1, f"{where}: tensor {i} has {t.numel()} elements, the plan {n}")


def _keep_alive(stream, *tensors) -> None:
    """Temporaries of an asynchronous call on a stream other than the current
    one stay allocated until that stream's work is done."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def compress_bound(ts: Tableset) -> int:
    b = C.c_uint64()
    _check(lib().zn_compress_bound(ts.handle, C.byref(b)), "compress_bound")
    return b.value


def scratch_bytes(ts: Tableset) -> int:
    b = C.c_uint64()
    _check(lib().zn_scratch_bytes(ts.handle, C.byref(b)), "scratch_bytes")
    return b.value


def new_scratch(ts: Tableset, device="cuda") -> torch.Tensor:
    return torch.empty(scratch_bytes(ts), dtype=torch.uint8, device=device)


def compress(ts: Tableset, tensors: Sequence[torch.Tensor], out: torch.Tensor | None = None,
             scratch: torch.Tensor | None = None, ptrs: torch.Tensor | None = None,
             sync: bool = True, stream=None):
    """zn_compress.  Returns the container (a view of `out`) when sync, else
    `out` itself (size at byte 56 once the stream has run)."""
    return compress2(ts, CODER_HUFFMAN, tensors, out, scratch, ptrs, sync, stream)


def compress2(ts: Tableset, coder: int, tensors: Sequence[torch.Tensor], out: torch.Tensor | None = None,
              scratch: torch.Tensor | None = None, ptrs: torch.Tensor | None = None,
              sync: bool = True, stream=None):
    """zn_compress2: compress with the exponent stream's coder chosen
    (CODER_HUFFMAN or CODER_TANS)."""
    _check_tensors(ts, tensors, "compress", exact=True)
    dev = tensors[0].device
    tmp = []
    if out is None:
        out = torch.empty(compress_bound(ts), dtype=torch.uint8, device=dev)
    if scratch is None:
        scratch = new_scratch(ts, dev)
        tmp.append(scratch)
    if ptrs is None:
        ptrs = _ptr_array(tensors, dev, stream)
        tmp.append(ptrs)
    for name, b in (("out", out), ("scratch", scratch)):
        if b.device != dev or not b.is_contiguous() or b.dtype != torch.uint8:
            raise ZnError(-1, f"compress: {name} must be a contiguous uint8 tensor on {dev}")
    if not sync:
        _keep_alive(stream, *tmp)
    nb = C.c_uint64()
    with torch.cuda.device(dev):   # the tableset must live on the tensors' device
        _check(lib().zn_compress2(ts.handle, int(coder), C.c_void_p(ptrs.data_ptr()),
                                  C.c_void_p(out.data_ptr()), out.numel(), C.byref(nb) if sync else None,
                                  C.c_void_p(scratch.data_ptr()), scratch.numel(), _stream(stream)),
               "compress")
    return out[: nb.value] if sync else out


def decompress(ts: Tableset, blob: torch.Tensor, outs: Sequence[torch.Tensor] | None = None,
               scratch: torch.Tensor | None = None, ptrs: torch.Tensor | None = None,
               sync: bool = True, stream=None):
    """zn_decompress into `outs` (allocated from the plan when None)."""
    if not blob.is_cuda or not blob.is_contiguous() or blob.dtype != torch.uint8:
        raise ZnError(-1, "decompress: the container must be a contiguous uint8 CUDA tensor")
    if outs is None:
        info = ts.info()
        outs = [torch.empty(n, dtype=TORCH_DTYPE[info["dtype"]], device=blob.device)
                for n in info["n_elems"]]
    _check_tensors(ts, outs, "decompress", exact=False)
    if outs and outs[0].device != blob.device:
        raise ZnError(-1, "decompress: outputs and container on different devices")
    tmp = []
    if scratch is None:
        scratch = torch.empty(256, dtype=torch.uint8, device=blob.device)
        tmp.append(scratch)
    if ptrs is None:
        ptrs = _ptr_array(outs, blob.device, stream)
        tmp.append(ptrs)
    if not sync:
        _keep_alive(stream, *tmp)
    with torch.cuda.device(blob.device):
        _check(lib().zn_decompress(ts.handle, C.c_void_p(blob.data_ptr()), blob.numel(),
                                   C.c_void_p(ptrs.data_ptr()), C.c_void_p(scratch.data_ptr()),
                                   scratch.numel(), 1 if sync else 0, _stream(stream)), "decompress")
    return outs


def decompress_noalloc(ts: Tableset, blob: torch.Tensor, outs: Sequence[torch.Tensor],
                       ptrs: torch.Tensor, status: torch.Tensor | None = None, sync: bool = True,
                       stream=None):
    """zn_decompress_noalloc: the library allocates nothing; the caller
    passes the outputs, their device pointer array and optionally a device
    int32 `status` that receives the error word."""
    if not blob.is_cuda or not blob.is_contiguous() or blob.dtype != torch.uint8:
        raise ZnError(-1, "decompress_noalloc: the container must be a contiguous uint8 CUDA tensor")
    _check_tensors(ts, outs, "decompress_noalloc", exact=False)
    if ptrs.device != blob.device or ptrs.dtype != torch.int64 or ptrs.numel() != len(outs):
        raise ZnError(-1, "decompress_noalloc: ptrs must be the outputs' int64 device pointers")
    if status is not None and (status.device != blob.device or status.dtype != torch.int32):
        raise ZnError(-1, "decompress_noalloc: status must be an int32 tensor on the container's device")
    with torch.cuda.device(blob.device):
        _check(lib().zn_decompress_noalloc(ts.handle, C.c_void_p(blob.data_ptr()), blob.numel(),
                                           C.c_void_p(ptrs.data_ptr()),
                                           C.c_void_p(status.data_ptr()) if status is not None else None,
                                           1 if sync else 0, _stream(stream)), "decompress_noalloc")
    return outs


def debug_histograms(ts: Tableset, tensors: Sequence[torch.Tensor], stream=None) -> torch.Tensor:
    info = ts.info()
    nc = {BF16: 1, FP32: 4, FP8_E4M3: 2, FP4X2_E2M1: 2}[info["dtype"]]
    hist = torch.zeros((info["n_chunks"], nc, 256), dtype=torch.int32, device=tensors[0].device)
    ptrs = _ptr_array(tensors, tensors[0].device)
    _check(lib().zn_debug_histograms(ts.handle, C.c_void_p(ptrs.data_ptr()),
                                     C.c_void_p(hist.data_ptr()), _stream(stream)), "histograms")
    torch.cuda.synchronize()
    return hist


def debug_code_lengths(hist: torch.Tensor, alphabet: int = 256, group_rule: bool = False,
                       stream=None) -> torch.Tensor:
    """Device package-merge of n histograms (int64 [n, 256] on the GPU)."""
    hist = hist.to(torch.int64).contiguous()
    out = torch.zeros(hist.shape, dtype=torch.uint8, device=hist.device)
    _check(lib().zn_debug_code_lengths(C.c_void_p(hist.data_ptr()), hist.shape[0], alphabet,
                                       1 if group_rule else 0, C.c_void_p(out.data_ptr()),
                                       _stream(stream)), "code_lengths")
    torch.cuda.synchronize()
    return out


def debug_kernel_events(kernel: str, before=None, after=None) -> None:
    """zn_debug_kernel_events with torch.cuda.Event objects (None stops the
    recording for that kernel).  Events not yet created are created here."""
    def handle(e):
        if e is None:
            return None
        if not e.cuda_event:
            e.record()
        return C.c_void_p(e.cuda_event)
    _check(lib().zn_debug_kernel_events(kernel.encode(), handle(before), handle(after)),
           "kernel_events")
