"""Helpers shared by the GPU tests: generation, oracle comparison, sampling."""
from __future__ import annotations

import numpy as np
import torch

from lossless_float_weight_amd import workloads as W
from lossless_float_weight_amd import zn

NP_DTYPE = {zn.BF16: np.uint16, zn.FP32: np.uint32, zn.FP8_E4M3: np.uint8, zn.FP4X2_E2M1: np.uint8}


def to_np(t: torch.Tensor) -> np.ndarray:
    return W.bits(t.contiguous()).reshape(-1).cpu().numpy()


def gpu_compress(tensors, chunk_bytes=262144, ts=None, n_groups=0):
    if ts is None:
        ts = zn.setup(tensors, chunk_bytes=chunk_bytes, n_groups=n_groups)
    blob = zn.compress(ts, tensors)
    torch.cuda.synchronize()
    return ts, blob


def assert_roundtrip(ts, blob, tensors):
    outs = zn.decompress(ts, blob)
    torch.cuda.synchronize()
    for a, b in zip(tensors, outs):
        assert torch.equal(W.bits(a.contiguous()).reshape(-1), W.bits(b).reshape(-1)), "round trip"


def first_difference(a: np.ndarray, b: np.ndarray) -> str:
    n = min(a.size, b.size)
    idx = np.nonzero(a[:n] != b[:n])[0]
    where = int(idx[0]) if idx.size else n
    return f"sizes {a.size} vs {b.size}, first differing byte {where}"


def record_bounds(blob: np.ndarray):
    """Directory of a container: (off_dir, n_chunks, offsets[n_chunks + 1])."""
    n_chunks = int(np.frombuffer(blob[24:28].tobytes(), np.uint32)[0])
    off_dir = int(np.frombuffer(blob[40:48].tobytes(), np.uint64)[0])
    dirv = np.frombuffer(blob[off_dir:off_dir + 8 * (n_chunks + 1)].tobytes(), np.uint64)
    return off_dir, n_chunks, dirv.astype(np.int64)


def field_modes(blob: np.ndarray, n_fields: int, kbits):
    """Per chunk, the tuple of its streams' modes (0 raw, 1 constant, 2 Huffman,
    3 group, 4 tANS) read from the records (format: 8-byte stream head, code
    lengths as nibbles when Huffman, a presence mask and the present symbols'
    u16 counts when tANS, u16 segment bit lengths when coded, then the 16-byte
    aligned payload)."""
    _, n_chunks, dirv = record_bounds(blob)
    out = []
    for c in range(n_chunks):
        pos, modes = int(dirv[c]), []
        for p in range(n_fields):
            h0 = int(np.frombuffer(blob[pos:pos + 4].tobytes(), np.uint32)[0])
            pay = int(np.frombuffer(blob[pos + 4:pos + 8].tobytes(), np.uint32)[0])
            mode, nseg = h0 & 0xFF, h0 >> 16
            head = 8 + ((1 << kbits[p]) // 2 if mode == 2 else 0) + (2 * nseg if mode in (2, 3) else 0)
            if mode == 4:
                A = 1 << kbits[p]
                d = sum(bin(int(v)).count("1") for v in blob[pos + 8:pos + 8 + A // 8])
                head = 8 + A // 8 + 2 * d + 2 * nseg
            pos += ((head + 15) & ~15) + ((pay + 15) & ~15)
            modes.append(mode)
        out.append(tuple(modes))
    return out


def oracle_compress_async(oracle, dt, arrs, chunk_bytes, ots=None):
    """The oracle's container of arrs, computed in a host thread (the oracle's
    C code runs with the interpreter lock released, so the GPU side of a test
    proceeds meanwhile).  Returns a future."""
    import concurrent.futures as cf
    ex = cf.ThreadPoolExecutor(1)
    fut = ex.submit(oracle.compress, dt, arrs, chunk_bytes, ots)
    ex.shutdown(wait=False)
    return fut
