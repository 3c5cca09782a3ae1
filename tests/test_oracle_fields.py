"""Oracle pins for the field split (exponent extraction) and merge.

The split follows THEORY-599 (nucleation note on ZipNN), per-field
compressibility (ZipNN Table II): the exponent is taken out, the sign and
fraction bytes stay as they are; FP8 follows "Lossless Compression of Neural
Network Components ... Low-Precision Formats", Abstract (exponent and
mantissa separated), and so does FP4 (E2M1, the same page's other format),
stored two values to a byte.  Pins: merge(split(x)) == x on every BF16, FP8
and FP4-pair bit pattern; the extracted field equals the IEEE-754 biased
exponent that numpy / torch report for normal numbers (frexp), and for FP4
the exponent and mantissa of each value of the E2M1 magnitude list (0, 0.5,
1, 1.5, 2, 3, 4, 6: bias 1, one mantissa bit, subnormals below 1);
hand-checked bit patterns.
"""
import numpy as np
import pytest
import torch

from tests import ref_tiny


def test_bf16_exhaustive_identity(oracle):
    x = np.arange(1 << 16, dtype=np.uint16)
    planes, raw = oracle.split(oracle.BF16, x)
    assert np.array_equal(oracle.merge(oracle.BF16, planes, raw), x)
    # every (E, SF) pair occurs exactly once: the split is a bijection
    key = planes[0].astype(np.int64) * 256 + raw
    assert np.unique(key).size == 1 << 16


def test_fp8_exhaustive_identity(oracle):
    x = np.arange(256, dtype=np.uint8)
    planes, raw = oracle.split(oracle.FP8_E4M3, x)
    assert np.array_equal(oracle.merge(oracle.FP8_E4M3, planes, raw), x)
    assert planes[0].max() == 15 and planes[1].max() == 7 and raw.max() == 1


def test_fp4_exhaustive_identity(oracle):
    x = np.arange(256, dtype=np.uint8)
    planes, raw = oracle.split(oracle.FP4X2_E2M1, x)
    assert np.array_equal(oracle.merge(oracle.FP4X2_E2M1, planes, raw), x)
    assert planes[0].max() == 15 and planes[1].max() == 3 and raw.max() == 3
    key = (planes[0].astype(np.int64) * 4 + planes[1]) * 4 + raw
    assert np.unique(key).size == 256          # a bijection


E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp4_fields_against_e2m1_values(oracle):
    # Each byte holds two values, the first in its low nibble; a nibble is a
    # sign bit over a 3-bit magnitude code.  From each value's magnitude
    # alone: exponent = 0 below 1 (subnormal), else floor(log2 |v|) + 1 (bias
    # 1); mantissa = the fraction's one bit (0.5 steps for subnormals).
    x = np.arange(256, dtype=np.uint8)
    planes, raw = oracle.split(oracle.FP4X2_E2M1, x)
    for half, shift in ((0, 0), (1, 4)):
        nib = (x >> shift) & 15
        mag = np.array([E2M1_MAGNITUDES[v & 7] for v in nib])
        neg = nib >= 8
        sub = mag < 1.0
        e = np.where(sub, 0, _frexp_exponent(np.where(sub, 1.0, mag)))
        m = np.where(sub, mag / 0.5, (mag / 2.0 ** (e - 1) - 1.0) * 2.0)
        assert np.array_equal((planes[0] >> (2 * half)) & 3, e.astype(np.uint8))
        assert np.array_equal((planes[1] >> half) & 1, m.astype(np.uint8))
        assert np.array_equal((raw >> half) & 1, neg.astype(np.uint8))


@pytest.mark.parametrize("value,e,m,s", [(0x21, 4, 1, 0), (0xF7, 15, 3, 2), (0x00, 0, 0, 0),
                                          (0x8A, 1, 0, 3), (0x1C, 2, 2, 1)])
def test_fp4_hand_checked(oracle, value, e, m, s):
    # 0x21: 0.5 then 1.0; 0xF7: 6.0 then -6.0; 0x8A: -1.0 then -0.0;
    # 0x1C: -2.0 then 0.5
    planes, raw = oracle.split(oracle.FP4X2_E2M1, np.array([value], np.uint8))
    assert (planes[0][0], planes[1][0], raw[0]) == (e, m, s)
    assert ref_tiny.split(3, value) == ([e, m], s)


def test_fp32_random_and_special_identity(oracle):
    rng = np.random.default_rng(7)
    x = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001,
                         0x00000001, 0x807FFFFF, 0x3F800000, 0xFFFFFFFF], np.uint32)
    x = np.concatenate([x, specials])
    planes, raw = oracle.split(oracle.FP32, x)
    assert np.array_equal(oracle.merge(oracle.FP32, planes, raw), x)


def _frexp_exponent(v):
    _, e = np.frexp(v)
    return e


def test_bf16_exponent_is_ieee_biased_exponent(oracle):
    x = np.arange(1 << 16, dtype=np.uint16)
    planes, raw = oracle.split(oracle.BF16, x)
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    normal = np.isfinite(f) & (np.abs(f) >= np.finfo(np.float32).tiny)
    assert np.array_equal(planes[0][normal].astype(np.int64) - 127, _frexp_exponent(f[normal]) - 1)
    # the raw byte holds the sign in its top bit and the top 7 fraction bits below
    assert np.array_equal(raw >> 7, (x >> 15).astype(np.uint8))
    assert np.array_equal(raw & 0x7F, (x & 0x7F).astype(np.uint8))


def test_fp32_planes_against_ieee(oracle):
    rng = np.random.default_rng(8)
    f = rng.standard_normal(1 << 16).astype(np.float32) * np.float32(3e3)
    x = f.view(np.uint32)
    planes, _ = oracle.split(oracle.FP32, x)
    assert np.array_equal(planes[0].astype(np.int64) - 127, _frexp_exponent(f.astype(np.float64)) - 1)
    frac = x & 0x7FFFFF
    assert np.array_equal(planes[1] & 0x7F, (frac >> 16).astype(np.uint8))
    assert np.array_equal(planes[1] >> 7, (x >> 31).astype(np.uint8))
    assert np.array_equal(planes[2], ((frac >> 8) & 0xFF).astype(np.uint8))
    assert np.array_equal(planes[3], (frac & 0xFF).astype(np.uint8))


def test_fp8_exponent_against_torch_e4m3(oracle):
    x = np.arange(256, dtype=np.uint8)
    planes, raw = oracle.split(oracle.FP8_E4M3, x)
    f = torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    normal = np.isfinite(f) & (np.abs(f) >= 2.0 ** -6)
    assert np.array_equal(planes[0][normal].astype(np.int64) - 7, _frexp_exponent(f[normal]) - 1)
    assert np.array_equal(raw.astype(bool), np.signbit(f) | (x >= 128))


@pytest.mark.parametrize("value,e,sf", [(0x3F80, 127, 0x00), (0xC000, 128, 0x80),
                                        (0x3F81, 127, 0x01), (0x0001, 0, 0x01),
                                        (0x7F80, 255, 0x00), (0xFFFF, 255, 0xFF)])
def test_bf16_hand_checked(oracle, value, e, sf):
    planes, raw = oracle.split(oracle.BF16, np.array([value], np.uint16))
    assert (planes[0][0], raw[0]) == (e, sf)
    # the independent pure-Python restatement agrees
    assert ref_tiny.split(0, value) == ([e], sf)
