"""The decompression entry point that allocates nothing, through the C ABI:
its outputs equal zn_decompress's (bit for bit) on two calls in a row, the
second with a smaller container, and its error reporting matches."""
import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from lossless_float_weight_amd import zn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zn.lib()


def _case(tensors, chunk_bytes, n_groups=0, coder=zn.CODER_HUFFMAN, pairs=False):
    ts = zn.setup(tensors, chunk_bytes=chunk_bytes, n_groups=n_groups, pairs=pairs)
    blob = zn.compress2(ts, coder, tensors)
    ref = zn.decompress(ts, blob)
    outs = [torch.full_like(r, 0) for r in ref]
    ptrs = torch.tensor([o.data_ptr() for o in outs], dtype=torch.int64, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    return ts, blob, ref, outs, ptrs, status


def _paired(n, seed):
    """BF16 values whose aligned pairs mostly repeat one exponent."""
    rng = np.random.default_rng(seed)
    e = 120 + np.minimum(rng.geometric(0.45, n), 8).astype(np.int64)
    same = rng.random(n) < 0.9
    e[1::2] = np.where(same[1::2], e[0::2][: e[1::2].size], e[1::2])
    x = (rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)
    return torch.from_numpy(x.astype(np.int32)).to(torch.int16).view(torch.bfloat16).cuda()


def test_noalloc_equals_decompress_twice_then_smaller():
    print("case: no-alloc decompression, BF16 block then smaller FP8 and BF16 tensors (Huffman, groups, "
          "packed pairs, tANS)", flush=True)
    big = _case([t for _, t in W.block_bf16("cuda", seed=2, scale=8)], 262144)
    small8 = _case([W.fp8_blockscaled(70001, device="cuda")[0][1]], 16384)
    small = _case([W.single_bf16(5000, device="cuda")[0][1]], 8192, n_groups=2)
    paired = _case([_paired(40001, 3)], 8192, n_groups=2, pairs=True)
    assert any(paired[0].pairs(g)[0] for g in range(2))
    tans = _case([W.single_bf16(3000, device="cuda")[0][1]], 4096, coder=zn.CODER_TANS)
    for ts, blob, ref, outs, ptrs, status in (big, small8, small, paired, tans):
        for sync in (True, False):
            for o in outs:
                o.zero_()
            zn.decompress_noalloc(ts, blob, outs, ptrs, status, sync=sync)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            for o, r in zip(outs, ref):
                assert torch.equal(W.bits(o), W.bits(r))


def test_noalloc_reports_corruption():
    print("case: no-alloc decompression of damaged containers", flush=True)
    ts, blob, ref, outs, ptrs, status = _case([W.single_bf16(50000, device="cuda")[0][1]], 16384)
    bad = blob.clone()
    bad[0] ^= 0xFF
    with pytest.raises(zn.ZnError) as e:
        zn.decompress_noalloc(ts, bad, outs, ptrs, status, sync=True)
    assert e.value.code == -2 and int(status.item()) == 2
    status.fill_(-1)
    zn.decompress_noalloc(ts, bad, outs, ptrs, status, sync=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    # a good call after the bad ones finds the shared control area reset
    zn.decompress_noalloc(ts, blob, outs, ptrs, status, sync=True)
    assert int(status.item()) == 0
    assert torch.equal(W.bits(outs[0]), W.bits(ref[0]))
    # the binding checks shapes before any launch
    with pytest.raises(zn.ZnError):
        zn.decompress_noalloc(ts, blob, [outs[0][:10]], ptrs, status)
