"""GPU parity of the tANS exponent coder: libzn.so (zn_compress2 with
ZN_CODER_TANS, and zn_decompress of such containers) against the CPU oracle.

THEORY-599's order-0 discussion (after ZipNN Fig. 4) names an FSE (tabled
ANS) coder as the exponent coder that beats Huffman by 0-2%; the oracle fixes
our reading of it.  The bar is the same as for Huffman: containers identical
to the oracle's byte for byte, exact round trips, the oracle's containers
decoded exactly, and damaged containers refused exactly when the oracle
refuses them.
"""
import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from lossless_float_weight_amd import zn
from tests.gpu_util import assert_roundtrip, field_modes, first_difference, to_np
from tests.test_gpu_parity import _fp32_mixes, _fp4_bytes

pytestmark = pytest.mark.gpu

ODT = {zn.BF16: 0, zn.FP32: 1, zn.FP8_E4M3: 2, zn.FP4X2_E2M1: 3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zn.lib()


def _tans(tensors, chunk_bytes):
    ts = zn.setup(tensors, chunk_bytes=chunk_bytes)
    blob = zn.compress2(ts, zn.CODER_TANS, tensors)
    torch.cuda.synchronize()
    return ts, blob


def _check(oracle, tensors, chunk_bytes, label):
    print(f"case: tANS {label} chunk={chunk_bytes}", flush=True)
    ts, blob = _tans(tensors, chunk_bytes)
    g = blob.cpu().numpy()
    o = oracle.compress(ODT[ts.dtype], [to_np(t) for t in tensors], chunk_bytes, coder=oracle.CODER_TANS)
    assert g.size == o.size and np.array_equal(g, o), first_difference(g, o)
    assert_roundtrip(ts, blob, tensors)
    # the oracle's container decodes on the GPU to the same tensors
    outs = zn.decompress(ts, torch.from_numpy(o).cuda())
    torch.cuda.synchronize()
    for a, b in zip(tensors, outs):
        assert torch.equal(W.bits(a.contiguous()).reshape(-1), W.bits(b).reshape(-1))
    return ts, g


def _modes0(blob, kb):
    """Mode of the first stream of every chunk."""
    from tests.gpu_util import record_bounds
    _, m, dirv = record_bounds(blob)
    return [int(blob[int(dirv[c])]) for c in range(m)]


@pytest.mark.parametrize("n", [1, 33, 511, 513, 4097, 131071, 131073, 300001])
@pytest.mark.parametrize("cb", [4096, 262144])
def test_bf16_ragged(oracle, n, cb):
    x = W.gaussian(n, 0.0, 0.02, torch.bfloat16, "cuda", seed=n, i=3)
    _check(oracle, [x], cb, f"BF16 n={n}")


def test_bf16_single_tensor_and_modes(oracle):
    x = W.single_bf16(device="cuda")[0][1]
    ts, g = _check(oracle, [x], 262144, "single BF16 2^20")
    assert set(_modes0(g, 8)) == {4}
    # constant, all bit patterns (near-uniform exponents: raw), a dominant
    # exponent with rare others (symbols of zero bits), one element
    gen = torch.Generator(device="cpu").manual_seed(5)
    const = torch.full((70000,), 1.0, dtype=torch.bfloat16, device="cuda")
    allp = torch.randperm(1 << 16, generator=gen).to(torch.int32).to(torch.int16).view(torch.bfloat16).cuda()
    dom = torch.full((50000,), 1.5, dtype=torch.bfloat16)
    dom[torch.randint(0, 50000, (40,), generator=gen)] = 3.0
    one = torch.tensor([-2.5], dtype=torch.bfloat16, device="cuda")
    ts, g = _check(oracle, [const, allp, dom.cuda(), one], 8192, "BF16 constant/patterns/dominant")
    modes = _modes0(g, 8)
    assert 1 in modes and 0 in modes and 4 in modes


def test_bf16_block_scaled(oracle):
    tensors = [t for _, t in W.block_bf16("cuda", seed=2, scale=4)]
    _check(oracle, tensors, 262144, "BF16 block / 4")


def test_bf16_unaligned_input(oracle):
    base = W.gaussian(40001, 0.0, 0.02, torch.bfloat16, "cuda", 9, 0)
    _check(oracle, [base[1:]], 16384, "BF16 unaligned view")


@pytest.mark.parametrize("n", [1, 1000, 65537, 300000])
def test_fp32(oracle, n):
    tensors = [t for _, t in W.fp32_pair(n, device="cuda")]
    _check(oracle, tensors, 262144 if n > 1000 else 4096, f"FP32 pair n={n}")


@pytest.mark.parametrize("n", [1, 1023, 1025, 262145, 600000])
def test_fp8(oracle, n):
    if n >= 128:
        x = W.fp8_blockscaled(n, device="cuda")[0][1]
    else:
        gen = torch.Generator(device="cpu").manual_seed(n)
        x = torch.randint(0, 256, (n,), generator=gen, dtype=torch.uint8).view(torch.float8_e4m3fn).cuda()
    _check(oracle, [x], 262144, f"FP8 n={n}")


@pytest.mark.parametrize("n", [3, 4097, 300001])
def test_fp4(oracle, n):
    x = W.fp4_blockscaled(2 * n, device="cuda")[0][1][:n].contiguous()
    _check(oracle, [x], 16384, f"FP4 pairs n={n}")


def test_largest_chunks(oracle):
    # 1 MiB chunks: 1024 segments per stream, the most a chunk has
    x = W.gaussian(3 * (1 << 19) + 77, 0.0, 0.02, torch.bfloat16, "cuda", seed=4, i=2)
    _check(oracle, [x], 1 << 20, "BF16 1 MiB chunks")
    y = W.fp8_blockscaled((1 << 21) + 5, device="cuda")[0][1]
    _check(oracle, [y], 1 << 20, "FP8 1 MiB chunks")


def test_grouped_plan_refuses_tans():
    tensors = [t for _, t in W.block_bf16("cuda", seed=2, scale=16)]
    ts = zn.setup(tensors, chunk_bytes=65536, n_groups=4)
    with pytest.raises(zn.ZnError) as e:
        zn.compress2(ts, zn.CODER_TANS, tensors)
    assert e.value.code == -1
    ts0 = zn.setup(tensors, chunk_bytes=65536)
    with pytest.raises(zn.ZnError):
        zn.compress2(ts0, 7, tensors)


def test_sizes_beat_huffman_by_the_pages_band(oracle):
    # ZipNN Fig. 4 / THEORY-599: 0-2% smaller exponent streams
    x = W.single_bf16(device="cuda")[0][1]
    ts = zn.setup([x])
    h = zn.compress(ts, [x]).numel()
    t = zn.compress2(ts, zn.CODER_TANS, [x]).numel()
    raw_sf = x.numel()   # the sign|fraction bytes, stored raw either way
    gain = 1 - (t - raw_sf) / (h - raw_sf)
    print(f"  exponent records: Huffman {h - raw_sf} B, tANS {t - raw_sf} B, gain {gain:.4f}", flush=True)
    assert 0.0 < gain <= 0.02


def test_damaged_tans_containers_decode_as_the_oracle_says(oracle):
    print("case: damaged tANS containers", flush=True)
    rng = np.random.default_rng(11)
    cases = []
    x = W.gaussian(20000, 0.0, 0.02, torch.bfloat16, "cuda", seed=3, i=4)
    cases.append(("bf16", x))
    y = W.fp8_blockscaled(30000, device="cuda")[0][1]
    cases.append(("fp8", y))
    for name, t in cases:
        ts, blob = _tans([t], 8192)
        g = blob.cpu().numpy()
        from tests.gpu_util import record_bounds
        off_dir, m, dirv = record_bounds(g)
        # flips inside the first stream's head (mask, counts, segment
        # lengths) and payload, where the tANS checks live, plus anywhere
        spots = []
        for c in range(m):
            r0 = int(dirv[c])
            spots += [r0 + int(v) for v in rng.integers(8, 96, 4)]
            spots += [r0 + int(v) for v in rng.integers(96, int(dirv[c + 1]) - r0, 2)]
        spots += [int(v) for v in rng.integers(64, g.size - 16, 6)]
        for sp in spots:
            bad = g.copy()
            bad[sp] ^= np.uint8(1 << int(rng.integers(0, 8)))
            est = oracle.decompress_status(bad, [t.numel()])
            out = torch.empty_like(t)
            try:
                zn.decompress(ts, torch.from_numpy(bad).cuda(), [out])
                torch.cuda.synchronize()
                st = 0
            except zn.ZnError as e:
                st = e.code
            assert st == est, f"{name} byte {sp}: GPU {st}, oracle {est}"
            if st == 0:
                want = oracle.decompress(bad, [t.numel()])[0]
                assert np.array_equal(to_np(out), want), f"{name} byte {sp}: outputs differ"


def test_block_full_size_whole_container(oracle):
    print("case: tANS 8B-shaped BF16 block, full size, whole-container parity", flush=True)
    import time
    t0 = time.time()
    tensors = [t for _, t in W.block_bf16("cuda", seed=2)]
    arrs = [to_np(t) for t in tensors]
    import concurrent.futures as cf
    ex = cf.ThreadPoolExecutor(1)
    fut = ex.submit(oracle.compress, oracle.BF16, arrs, 262144, None, False, oracle.CODER_TANS)
    ex.shutdown(wait=False)
    ts, blob = _tans(tensors, 262144)
    g = blob.cpu().numpy()
    print(f"  GPU container {g.size} bytes at {time.time() - t0:.0f} s", flush=True)
    assert_roundtrip(ts, blob, tensors)
    del blob
    while True:
        try:
            o = fut.result(timeout=30)
            break
        except cf.TimeoutError:
            print(f"  oracle still running at {time.time() - t0:.0f} s", flush=True)
    print(f"  oracle container {o.size} bytes at {time.time() - t0:.0f} s", flush=True)
    assert g.size == o.size and np.array_equal(g, o), first_difference(g, o)


def test_fp8_full_size_whole_container(oracle):
    # the 2^30-value block-scaled FP8 tensor: both coded streams may take tANS
    # lanes beside raw ones; the oracle works on the host meanwhile
    print("case: tANS FP8 E4M3 2^30, whole-container parity", flush=True)
    import time
    t0 = time.time()
    tensors = [W.fp8_blockscaled(1 << 30, device="cuda")[0][1]]
    arrs = [to_np(t) for t in tensors]
    import concurrent.futures as cf
    ex = cf.ThreadPoolExecutor(1)
    fut = ex.submit(oracle.compress, oracle.FP8_E4M3, arrs, 262144, None, False, oracle.CODER_TANS)
    ex.shutdown(wait=False)
    ts, blob = _tans(tensors, 262144)
    g = blob.cpu().numpy()
    print(f"  GPU container {g.size} bytes at {time.time() - t0:.0f} s", flush=True)
    assert_roundtrip(ts, blob, tensors)
    del blob
    while True:
        try:
            o = fut.result(timeout=30)
            break
        except cf.TimeoutError:
            print(f"  oracle still running at {time.time() - t0:.0f} s", flush=True)
    print(f"  oracle container {o.size} bytes at {time.time() - t0:.0f} s", flush=True)
    assert g.size == o.size and np.array_equal(g, o), first_difference(g, o)


def test_every_decode_path_with_tans_lanes(oracle):
    # tANS exponent lanes next to Huffman lanes of the other streams in the
    # same wave (FP32 16 lanes per stream, FP8 and FP4 32), and next to raw
    # and constant streams
    ts32 = [t.cuda() for t in _fp32_mixes()] + [W.gaussian(4096, 0.0, 0.02, torch.float32, "cuda", 9, 0)]
    _, g = _check(oracle, ts32, 16384, "FP32 field-mode mixes")
    m32 = set(field_modes(g, 4, [8, 8, 8, 8]))
    assert any(m[0] == 4 and m.count(2) == 3 for m in m32), m32
    assert any(m[0] == 4 and 0 in m[1:] for m in m32), m32
    gen = torch.Generator(device="cpu").manual_seed(8)
    n = 4096
    both = torch.randint(0, 6, (n,), generator=gen).to(torch.uint8) * 9
    e4 = W.fp8_blockscaled(n, device="cpu")[0][1].view(torch.uint8)
    ts8 = [x.view(torch.float8_e4m3fn).cuda() for x in (both, e4)]
    _, g = _check(oracle, ts8, 4096, "FP8 field-mode mixes")
    m8 = set(field_modes(g, 2, [4, 3]))
    assert (4, 2) in m8 and (4, 0) in m8, m8
    sk = lambda: torch.randint(0, 8, (n,), generator=gen).clamp(max=4) // 2        # noqa: E731
    few = lambda: (torch.randint(0, 8, (n,), generator=gen) == 0).to(torch.int64)  # noqa: E731
    bit = lambda: torch.randint(0, 2, (n,), generator=gen)                          # noqa: E731
    nib = lambda e, m, s: 8 * s + 2 * e + m                                         # noqa: E731
    ts4 = [_fp4_bytes(nib(sk(), few(), bit()), nib(sk(), few(), bit())).cuda(),
           _fp4_bytes(nib(sk(), bit(), bit()), nib(sk(), bit(), bit())).cuda()]
    _, g = _check(oracle, ts4, 4096, "FP4 field-mode mixes")
    m4 = set(field_modes(g, 2, [4, 2]))
    assert (4, 2) in m4 and (4, 0) in m4, m4


def test_empty_tensors(oracle):
    x = W.single_bf16(1000, device="cuda")[0][1]
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    _check(oracle, [e, x, e], 4096, "BF16 with empty tensors")
    _check(oracle, [e], 4096, "one empty BF16 tensor")
