"""Oracle pins for the whole container: lossless round trip, exact sizes,
order-0 invariances and the pages' printed ratios as plausibility bands.

Sources: "NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract
(exact bit-to-bit reconstruction); "Lossless Compression of Neural Network
Components ... Low-Precision Formats", Abstract (lossless; 83% for FP8);
THEORY-599 (nucleation note on ZipNN): per-field compressibility (ZipNN
Table II), order-0 only (ZipNN section III-A b), implied entropy, exponent
distribution (ZipNN Fig. 2).
"""
import json
import os

import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from tests import ref_tiny

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def _bits_np(t):
    return W.bits(t).cpu().numpy().ravel()


def _bf16(n, std=0.02, seed=0):
    return _bits_np(W.gaussian(n, 0.0, std, torch.bfloat16, "cpu", seed, 0))


def _roundtrip(oracle, dt, tensors, cb=262144, ts=None):
    blob = oracle.compress(dt, tensors, cb, ts)
    outs = oracle.decompress(blob, [t.size for t in tensors], dt, ts)
    for a, b in zip(tensors, outs):
        assert np.array_equal(a, b)
    return blob


# ------------------------------------------------------------- round trip --
@pytest.mark.parametrize("n", [1, 2, 511, 512, 513, 2047, 2048, 2049, 131071, 131072, 131073,
                               300000])
def test_roundtrip_bf16_ragged(oracle, n):
    _roundtrip(oracle, oracle.BF16, [_bf16(n, seed=n)], cb=262144)
    _roundtrip(oracle, oracle.BF16, [_bf16(n, seed=n)], cb=4096)


@pytest.mark.parametrize("dt", [0, 1, 2, 3])
def test_roundtrip_every_bit_pattern(oracle, dt):
    rng = np.random.default_rng(dt)
    if dt == 0:
        x = rng.permutation(np.arange(1 << 16, dtype=np.uint16))
    elif dt in (2, 3):
        x = np.tile(np.arange(256, dtype=np.uint8), 64)
    else:
        x = rng.integers(0, 1 << 32, 70000, dtype=np.uint64).astype(np.uint32)
    _roundtrip(oracle, dt, [x], cb=8192)


def test_roundtrip_multi_tensor_mixed_modes(oracle):
    rng = np.random.default_rng(9)
    tensors = [
        _bf16(5000, seed=1),
        np.full(7000, 0x3F80, np.uint16),                          # constant exponent
        rng.integers(0, 1 << 16, 9000, dtype=np.uint64).astype(np.uint16),  # random bits
        _bf16(1, seed=2),
        (_bits_np(W.gaussian(6000, 1.0, 0.05, torch.bfloat16, "cpu", 3, 0))),
    ]
    blob, st = oracle.compress(oracle.BF16, tensors, 4096, with_stats=True)
    outs = oracle.decompress(blob, [t.size for t in tensors])
    for a, b in zip(tensors, outs):
        assert np.array_equal(a, b)
    assert st["mode_count"][0][oracle.CONST] >= 4   # constant tensor + single-element tensor
    assert st["mode_count"][0][oracle.HUFF] >= 3


def test_roundtrip_fp8_and_fp32_configs_small(oracle):
    x8 = _bits_np(W.fp8_blockscaled(300000, device="cpu", seed=4)[0][1])
    _roundtrip(oracle, oracle.FP8_E4M3, [x8])
    pair = W.fp32_pair(150000, device="cpu", seed=3)
    _roundtrip(oracle, oracle.FP32, [_bits_np(t) for _, t in pair])
    x4 = W.fp4_blockscaled(300001, device="cpu", seed=8)[0][1].numpy()
    blob, st = oracle.compress(oracle.FP4X2_E2M1, [x4], 262144, with_stats=True)
    (y4,) = oracle.decompress(blob, [x4.size], oracle.FP4X2_E2M1)
    assert np.array_equal(x4, y4)
    # block-scaled values use every exponent, but not evenly: the exponent
    # pairs are coded below their 4 raw bits, the near-uniform mantissa bits
    # stay raw (the whole container is then about as large as the input)
    assert st["mode_count"][0][oracle.HUFF] > 0 and st["mode_count"][1][oracle.RAW] > 0
    assert st["payload_bits"][0] < 4 * x4.size


# -------------------------------------------------- independent restatement --
@pytest.mark.parametrize("dt,n", [(0, 3000), (0, 1), (1, 2500), (2, 5000), (3, 5001), (3, 3)])
def test_bytes_equal_independent_python_encoder(oracle, dt, n):
    rng = np.random.default_rng(n)
    if dt == 0:
        tensors = [_bf16(n, seed=5), np.full(100, 0x4000, np.uint16)]
    elif dt == 1:
        f = (rng.standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
        tensors = [f, f & np.uint32(0xFFFF0000)]
    elif dt == 2:
        tensors = [_bits_np(W.fp8_blockscaled(n, device="cpu", seed=6)[0][1])]
    else:
        tensors = [W.fp4_blockscaled(n, device="cpu", seed=9)[0][1].numpy(), np.full(77, 0x22, np.uint8)]
    blob = oracle.compress(dt, tensors, 4096)
    ref = ref_tiny.encode_container(dt, [[int(v) for v in t] for t in tensors], 4096)
    assert blob.tobytes() == ref
    dec = ref_tiny.decode_container(ref)
    for a, b in zip(tensors, dec):
        assert a.tolist() == b


# --------------------------------------------------------- exact sizes -----
def test_payload_bits_closed_form(oracle):
    x = _bf16(200000, seed=11)
    blob, st = oracle.compress(oracle.BF16, [x], 262144, with_stats=True)
    e = ((x >> 7) & 0xFF).astype(np.int64)
    bits = 0
    for c0 in range(0, x.size, 131072):
        h = np.bincount(e[c0:c0 + 131072], minlength=256)
        ln = ref_tiny.package_merge([int(v) for v in h])
        bits += int(np.dot(h, ln))
    assert st["payload_bits"][0] == bits


def test_within_chunk_permutation_keeps_size_exactly(oracle):
    x = _bf16(262144, seed=12)
    rng = np.random.default_rng(12)
    y = x.copy()
    for c0 in range(0, y.size, 131072):
        y[c0:c0 + 131072] = rng.permutation(y[c0:c0 + 131072])
    assert oracle.compress(oracle.BF16, [x]).size == oracle.compress(oracle.BF16, [y]).size


def test_global_shuffle_changes_ratio_little(oracle):
    x = _bf16(1 << 21, seed=13)
    y = np.random.default_rng(13).permutation(x)
    a, b = oracle.compress(oracle.BF16, [x]).size, oracle.compress(oracle.BF16, [y]).size
    assert abs(a - b) / a <= GOLDEN["shuffle_max_relative_change"]["value"]


# ------------------------------------------------ the pages' ratios (bands) --
def _frac(oracle, dt, tensors, esize):
    blob = oracle.compress(dt, tensors)
    return blob.size / sum(t.size * esize for t in tensors)


def test_ratio_bands_bf16_block(oracle):
    block = W.block_bf16("cpu", seed=2, scale=8)
    tensors = [_bits_np(t) for _, t in block]
    r = _frac(oracle, oracle.BF16, tensors, 2)
    lo, hi = GOLDEN["bf16_compressed_fraction"]["band"]
    assert lo <= r <= hi, r


def test_ratio_bands_fp32_and_clean(oracle):
    reg, clean = [_bits_np(t) for _, t in W.fp32_pair(1 << 19, device="cpu", seed=3)]
    r_reg = _frac(oracle, oracle.FP32, [reg], 4)
    r_clean = _frac(oracle, oracle.FP32, [clean], 4)
    lo, hi = GOLDEN["fp32_compressed_fraction"]["band"]
    assert lo <= r_reg <= hi, r_reg
    lo, hi = GOLDEN["clean_fp32_compressed_fraction"]["band"]
    assert lo <= r_clean <= hi, r_clean


def test_ratio_band_fp8(oracle):
    x = _bits_np(W.fp8_blockscaled(1 << 20, device="cpu", seed=4)[0][1])
    r = _frac(oracle, oracle.FP8_E4M3, [x], 1)
    lo, hi = GOLDEN["fp8_compressed_fraction"]["band"]
    assert lo <= r <= hi, r


def test_field_bands_and_exponent_statistics(oracle):
    x = _bf16(1 << 20, seed=14)
    blob, st = oracle.compress(oracle.BF16, [x], with_stats=True)
    exp_frac = st["stream_bytes"][0] / x.size
    lo, hi = GOLDEN["exponent_compressed_fraction"]["band"]
    assert lo <= exp_frac <= hi, exp_frac
    assert st["raw_plane_bytes"] / x.size == 1.0    # sign+fraction byte kept whole
    e = ((x >> 7) & 0xFF).astype(np.int64)
    h = np.bincount(e, minlength=256)
    top12 = np.sort(h)[::-1][:12].sum() / h.sum()
    lo, hi = GOLDEN["top12_exponent_coverage"]["band"]
    assert lo <= top12 <= hi
    lo, hi = GOLDEN["distinct_exponents_max"]["band"]
    assert lo <= np.count_nonzero(h) <= hi
    H = ref_tiny.entropy_bits([int(v) for v in h])
    lo, hi = GOLDEN["implied_entropy_bits"]["band"]
    assert lo <= H <= hi
    mean = st["payload_bits"][0] / x.size
    assert H <= mean < H + 1


def test_modes_follow_field_statistics(oracle):
    reg, clean = [_bits_np(t) for _, t in W.fp32_pair(1 << 17, device="cpu", seed=3)]
    _, st = oracle.compress(oracle.FP32, [reg], with_stats=True)
    assert st["mode_count"][0][oracle.HUFF] == 2          # exponent plane coded
    assert st["mode_count"][3][oracle.RAW] == 2           # low fraction byte raw
    _, st = oracle.compress(oracle.FP32, [clean], with_stats=True)
    assert st["mode_count"][2][oracle.CONST] == 2         # zeroed bytes are constant
    assert st["mode_count"][3][oracle.CONST] == 2


# ------------------------------------------------------------- corruption --
def test_corruption_never_crashes(oracle):
    x = _bf16(20000, seed=15)
    blob = oracle.compress(oracle.BF16, [x], 4096)
    rng = np.random.default_rng(15)
    results = set()
    for trial in range(400):
        b = blob.copy()
        kind = trial % 4
        if kind == 0:
            b = b[: int(rng.integers(0, b.size))]
        elif kind == 1:
            for _ in range(int(rng.integers(1, 6))):
                i = int(rng.integers(0, b.size))
                b[i] ^= np.uint8(1 << int(rng.integers(0, 8)))
        elif kind == 2:
            i = int(rng.integers(64, 64 + 16 + 8 * 11))
            b[i] = rng.integers(0, 256)
        else:
            i = int(rng.integers(0, 64))
            b[i] = rng.integers(0, 256)
        rc = oracle.decompress_status(b, [x.size])
        results.add(rc)
        assert rc in (0, -2, -4, -1)
    assert -2 in results


def test_corrupt_lengths_table_detected(oracle):
    x = _bf16(4096, seed=16)
    blob = oracle.compress(oracle.BF16, [x], 8192)
    off = int(np.frombuffer(blob[48:56].tobytes(), np.uint64)[0])
    assert blob[off] == oracle.HUFF
    b = blob.copy()
    b[off + 8:off + 8 + 128] = 0x11      # every symbol length 1: violates Kraft
    assert oracle.decompress_status(b, [x.size]) == -2
