"""GPU parity of packed exponent pairs ("NeuralZip: Reusable Setup for Fast
Lossless Compression", Abstract: recurring exponent tuples represented by
packed exponents, chosen by the setup), through the C ABI, against the oracle:
the setup (groups, F, token lengths, packing flags, saved bytes and hash),
containers byte for byte, exact round trips, the oracle's containers decoded on
the GPU, reuse on a perturbed copy with escapes, transfer, save and load, and
damaged containers refused as the oracle refuses them.
"""
import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from lossless_float_weight_amd import zn
from tests.gpu_util import first_difference, to_np
from tests.test_gpu_errors import _corruptions, _expected_status, _gpu_status

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zn.lib()


def _paired(n, seed, p_same=0.9):
    """BF16 values whose aligned pairs mostly repeat one exponent."""
    rng = np.random.default_rng(seed)
    e = 120 + np.minimum(rng.geometric(0.45, n), 8).astype(np.int64)
    same = rng.random(n) < p_same
    e[1::2] = np.where(same[1::2], e[0::2][: e[1::2].size], e[1::2])
    x = ((rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)).astype(np.int64)
    return torch.from_numpy(x.astype(np.int32)).to(torch.int16).view(torch.bfloat16).cuda()


def _same_setup(ts, ots, K):
    assert ts.group_map() == ots.group_map().tolist()
    for g in range(K):
        assert ts.lengths(g) == ots.lengths(g).tolist()
        packed, F, tl = ts.pairs(g)
        opk, oF, otl = ots.pairs(g)
        assert packed == opk and F == oF and tl == otl.tolist(), g
    assert ts.hash == ots.hash and ts.save() == ots.save()


def _check(oracle, tensors, cb, K, label, ts=None, ots=None):
    print(f"case: pairs {label} K={K} chunk={cb}", flush=True)
    if ts is None:
        ts = zn.setup(tensors, chunk_bytes=cb, n_groups=K, pairs=True)
        ots = oracle.setup(oracle.BF16, [to_np(t) for t in tensors], cb, K, pairs=True)
        _same_setup(ts, ots, K)
    blob = zn.compress(ts, tensors)
    torch.cuda.synchronize()
    g = blob.cpu().numpy()
    o = oracle.compress(oracle.BF16, [to_np(t) for t in tensors], cb, ots)
    assert g.size == o.size and np.array_equal(g, o), first_difference(g, o)
    for src in (blob, torch.from_numpy(o).cuda()):
        outs = zn.decompress(ts, src)
        torch.cuda.synchronize()
        for a, b in zip(tensors, outs):
            assert torch.equal(W.bits(a.contiguous()).reshape(-1), W.bits(b).reshape(-1))
    return ts, ots, g


def test_paired_data_packs_and_equals_oracle(oracle):
    tensors = [_paired(70001, 1), _paired(4097, 2, 0.6), _paired(1, 3), _paired(33, 4)]
    ts, ots, g = _check(oracle, tensors, 16384, 3, "repeating pairs, ragged")
    assert any(ts.pairs(i)[0] for i in range(3))


@pytest.mark.parametrize("cb", [4096, 262144])
def test_weights_equal_oracle(oracle, cb):
    tensors = [t for _, t in W.block_bf16("cuda", seed=2, scale=8)] + [_paired(300001, 5)]
    _check(oracle, tensors, cb, 8, "block / 8 + repeating pairs")


def test_unaligned_view_and_reuse_with_escapes(oracle):
    base = [_paired(50001, 7), _paired(20000, 8)]
    ts, ots, _ = _check(oracle, base, 8192, 2, "base")
    # the same setup on a same-shaped copy with new values (escapes) and an
    # unaligned view of the same size
    other = [b.clone() for b in base]
    v = other[0].view(torch.int16)
    v[::97] = (v[::97] & -32641) | (3 << 7)
    big = torch.cat([torch.zeros(1, dtype=torch.bfloat16, device="cuda"), base[1]])
    _check(oracle, [other[0], big[1:]], 8192, 2, "reuse with escapes, unaligned", ts, ots)


def test_transfer_save_and_load(oracle):
    src = [_paired(80000, 11)]
    ts = zn.setup(src, chunk_bytes=8192, n_groups=4, pairs=True)
    ots = oracle.setup(oracle.BF16, [to_np(t) for t in src], 8192, 4, pairs=True)
    _same_setup(ts, ots, 4)
    new = [_paired(33333, 12, 0.8)]
    tt = zn.setup_transfer(ts, new)
    ott = oracle.setup_transfer(ots, [to_np(t) for t in new])
    _same_setup(tt, ott, 4)
    _check(oracle, new, 8192, 4, "transferred", tt, ott)
    lt = zn.Tableset.load(ts.save())
    _check(oracle, src, 8192, 4, "loaded from saved bytes", lt, ots)
    lo = zn.Tableset.load(ots.save())
    _check(oracle, src, 8192, 4, "loaded from the oracle's bytes", lo, ots)


def test_damaged_pair_containers_decode_as_the_oracle_says(oracle):
    print("case: damaged pair containers", flush=True)
    tensors = [_paired(40000, 21), _paired(9001, 22, 0.7)]
    ts = zn.setup(tensors, chunk_bytes=8192, n_groups=2, pairs=True)
    ots = oracle.setup(oracle.BF16, [to_np(t) for t in tensors], 8192, 2, pairs=True)
    _same_setup(ts, ots, 2)
    assert any(ts.pairs(i)[0] for i in range(2))
    blob = zn.compress(ts, tensors).cpu().numpy()
    rng = np.random.default_rng(5)
    n_ok = 0
    for label, bad, _ in _corruptions(blob, rng, 48):
        want, wouts = _expected_status(oracle, bad, tensors, ots)
        got, gouts = _gpu_status(ts, bad, tensors, sync=True)
        assert got == want, f"{label}: GPU {got}, oracle {want}"
        if want == 0:
            n_ok += 1
            for a, b in zip(gouts, wouts):
                assert np.array_equal(to_np(a), b), f"{label}: outputs differ"
    print(f"  {n_ok} damaged containers still decode, as in the oracle", flush=True)


def test_model_scaled_with_pairs(oracle):
    # the 8B-shaped model at 1/16 scale with its KV cache, 16 groups with pairs
    named = W.model_bf16("cuda", seed=5, n_layers=2, scale=16, kv_tokens=2048)
    tensors = [t for _, t in named]
    ts, ots, g = _check(oracle, tensors, 262144, 16, "model / 16 (2 blocks, KV)")
    plain = zn.setup(tensors, chunk_bytes=262144, n_groups=16)
    pb = zn.compress(plain, tensors).numel()
    n_packed = sum(ts.pairs(i)[0] for i in range(16))
    print(f"  {n_packed} of 16 groups pack; container {g.size} bytes with pairs, {pb} without "
          f"({1 - g.size / pb:+.5f})", flush=True)


def test_empty_tensors_and_more_groups_than_chunks(oracle):
    # zero-element tensors beside others, and K larger than the chunk count
    # (empty groups: no F, never packing)
    cases = [([_paired(20001, 31), _paired(0, 32), _paired(5, 33)], 16384, 8, "empty tensor, K > chunks"),
             ([_paired(3, 34)], 4096, 4, "one chunk of 3 values")]
    for tensors, cb, K, label in cases:
        ts, ots, g = _check(oracle, tensors, cb, K, label)
        n_chunks = ts.info()["n_chunks"]
        used = set(ts.group_map())
        for i in range(K):
            if i not in used:
                packed, F, tl = ts.pairs(i)
                assert not packed and F == [] and not any(tl), i
        assert n_chunks < K


def test_all_empty_plan_with_pairs(oracle):
    print("case: pairs, every tensor empty", flush=True)
    tensors = [_paired(0, 41), _paired(0, 42)]
    ts = zn.setup(tensors, chunk_bytes=8192, n_groups=2, pairs=True)
    ots = oracle.setup(oracle.BF16, [to_np(t) for t in tensors], 8192, 2, pairs=True)
    _same_setup(ts, ots, 2)
    blob = zn.compress(ts, tensors)
    torch.cuda.synchronize()
    o = oracle.compress(oracle.BF16, [to_np(t) for t in tensors], 8192, ots)
    assert np.array_equal(blob.cpu().numpy(), o)
    outs = zn.decompress(ts, blob)
    assert all(x.numel() == 0 for x in outs)
