"""Lossless exponent-Huffman codec for floating-point tensors on AMD MI355X.

The GPU path is libzn.so (HIP kernels for gfx950, C ABI in include/zn.h);
`zn` is its Python binding and `workloads` the seeded synthetic inputs.
"""
from . import workloads  # noqa: F401
from . import zn  # noqa: F401
from .zn import (BF16, FP32, FP8_E4M3, FP4X2_E2M1, Tableset, ZnError, compress,  # noqa: F401
                 compress_bound, decompress, plan_from_container, scratch_bytes, setup, setup_transfer)
