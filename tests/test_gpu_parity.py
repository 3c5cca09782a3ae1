"""GPU parity: libzn.so (HIP kernels, through the C ABI) against the CPU oracle.

The bar is bit-exactness: container bytes identical to the oracle's on the
same seeded inputs, and decompressed tensors identical to the inputs.  Every
case, the full-size workloads included, compares whole containers.
"""
import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from lossless_float_weight_amd import zn
from tests.gpu_util import (assert_roundtrip, field_modes, first_difference, gpu_compress,
                            oracle_compress_async, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zn.lib()  # a missing library is an error wherever a GPU is present, not a skip


def _check_equal(oracle, dt, tensors, chunk_bytes, ts=None, ots=None):
    ts, blob = gpu_compress(tensors, chunk_bytes, ts)
    g = blob.cpu().numpy()
    o = oracle.compress(dt, [to_np(t) for t in tensors], chunk_bytes, ots)
    assert g.size == o.size and np.array_equal(g, o), first_difference(g, o)
    assert_roundtrip(ts, blob, tensors)
    return ts, blob


# ------------------------------------------------------------ BF16 ---------
def test_config1_single_bf16(oracle):
    print("case: single BF16 tensor 2^20, 256 KiB chunks", flush=True)
    x = W.single_bf16(device="cuda")[0][1]
    _check_equal(oracle, oracle.BF16, [x], 262144)


@pytest.mark.parametrize("n", [1, 7, 511, 512, 513, 2048, 4097, 131071, 131073, 300001])
@pytest.mark.parametrize("cb", [4096, 262144])
def test_bf16_ragged(oracle, n, cb):
    print(f"case: BF16 n={n} chunk={cb}", flush=True)
    x = W.gaussian(n, 0.0, 0.02, torch.bfloat16, "cuda", seed=n, i=1)
    _check_equal(oracle, oracle.BF16, [x], cb)


def test_bf16_every_pattern_and_modes(oracle):
    print("case: BF16 all bit patterns, constant, random, single element", flush=True)
    g = torch.Generator(device="cpu").manual_seed(3)
    perm = torch.randperm(1 << 16, generator=g)
    allp = perm.to(torch.int32).to(torch.int16).view(torch.bfloat16).cuda()
    const = torch.full((70000,), 1.0, dtype=torch.bfloat16, device="cuda")
    rnd = torch.randint(-32768, 32767, (90000,), generator=g, dtype=torch.int16).view(torch.bfloat16).cuda()
    one = torch.tensor([-2.5], dtype=torch.bfloat16, device="cuda")
    norm = W.gaussian(6000, 1.0, 0.05, torch.bfloat16, "cuda", 7, 0)
    _check_equal(oracle, oracle.BF16, [allp, const, rnd, one, norm], 8192)


def test_bf16_block_scaled(oracle):
    print("case: BF16 transformer block / 4", flush=True)
    tensors = [t for _, t in W.block_bf16("cuda", seed=2, scale=4)]
    _check_equal(oracle, oracle.BF16, tensors, 262144)


def test_bf16_unaligned_input(oracle):
    print("case: BF16 unaligned input view", flush=True)
    base = W.gaussian(40001, 0.0, 0.02, torch.bfloat16, "cuda", 9, 0)
    x = base[1:]  # 2-byte offset: the scalar path
    _check_equal(oracle, oracle.BF16, [x], 16384)


# ------------------------------------------------------- FP32 and FP8 ------
def test_fp32_regular_and_clean(oracle):
    print("case: FP32 regular + clean, 2^19 each", flush=True)
    tensors = [t for _, t in W.fp32_pair(1 << 19, device="cuda")]
    _check_equal(oracle, oracle.FP32, tensors, 262144)


@pytest.mark.parametrize("n", [1, 1000, 65537])
def test_fp32_ragged_and_random(oracle, n):
    print(f"case: FP32 random bits n={n}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(n)
    x = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), generator=g, dtype=torch.int32).view(torch.float32)
    y = W.gaussian(n, 0.0, 0.02, torch.float32, "cpu", n, 2)
    _check_equal(oracle, oracle.FP32, [x.cuda(), y.cuda()], 16384)


def _fp32_mixes():
    """One FP32 tensor per chunk (16 KiB chunks of 4096 values), each with
    another mix of coded, raw and constant field bytes."""
    g = torch.Generator(device="cpu").manual_seed(7)
    n = 4096
    small = torch.randint(0, 16, (n,), generator=g).to(torch.float32)          # 2 coded, 2 constant
    pick = torch.randn(23, generator=g)[torch.randint(0, 23, (n,), generator=g)]  # all 4 coded
    top = (torch.randint(0, 8, (n,), generator=g) << 16) | torch.randint(0, 1 << 16, (n,), generator=g)
    mixed = ((torch.randint(120, 124, (n,), generator=g) << 23) | top).to(torch.int32).view(torch.float32)
    sparse = torch.randint(0, 1 << 16, (n,), generator=g).to(torch.int32).view(torch.float32)  # 2 raw, 2 const
    return [small, pick, mixed, sparse]


def test_fp32_every_decode_path(oracle):
    # all coded; coded exponent + raw fraction; coded + raw + constant;
    # several coded streams with raw ones; raw and constant only
    print("case: FP32 field-mode mixes", flush=True)
    ts = [t.cuda() for t in _fp32_mixes()] + [W.gaussian(4096, 0.0, 0.02, torch.float32, "cuda", 9, 0)]
    _, blob = _check_equal(oracle, oracle.FP32, ts, 16384)
    modes = set(field_modes(blob.cpu().numpy(), 4, [8, 8, 8, 8]))
    assert (2, 2, 2, 2) in modes and (2, 0, 0, 0) in modes
    assert any(m.count(2) in (2, 3) and 0 in m for m in modes)
    assert any(1 in m and 2 in m for m in modes) and any(2 not in m for m in modes)


def test_fp8_every_decode_path(oracle):
    print("case: FP8 field-mode mixes", flush=True)
    g = torch.Generator(device="cpu").manual_seed(8)
    n = 4096
    both = torch.randint(0, 6, (n,), generator=g).to(torch.uint8) * 9          # E4 and M3 skewed: both coded
    m3 = (torch.randint(0, 16, (n,), generator=g) << 3 | torch.randint(0, 2, (n,), generator=g)).to(torch.uint8)
    e4 = W.fp8_blockscaled(n, device="cpu")[0][1].view(torch.uint8)             # E4 coded, M3 raw
    ts = [x.view(torch.float8_e4m3fn).cuda() for x in (both, m3, e4)]
    _, blob = _check_equal(oracle, oracle.FP8_E4M3, ts, 4096)
    modes = set(field_modes(blob.cpu().numpy(), 2, [4, 3]))
    assert (2, 2) in modes and (2, 0) in modes and (0, 2) in modes


def test_fp8_blockscaled(oracle):
    print("case: FP8 E4M3 block-scaled 2^20", flush=True)
    x = W.fp8_blockscaled(1 << 20, device="cuda")[0][1]
    _check_equal(oracle, oracle.FP8_E4M3, [x], 262144)


@pytest.mark.parametrize("n", [1, 15, 17, 2049, 70001])
def test_fp8_ragged_every_pattern(oracle, n):
    print(f"case: FP8 patterns n={n}", flush=True)
    x = (torch.arange(n, dtype=torch.int64) * 37 % 256).to(torch.uint8).view(torch.float8_e4m3fn)
    _check_equal(oracle, oracle.FP8_E4M3, [x.cuda()], 4096)


@pytest.mark.parametrize("dt", ["fp8", "fp4"])
def test_1byte_mantissa_raw_whole_segments(oracle, dt):
    # chunks of whole 1024-element segments, exponent coded and mantissa raw:
    # the mantissa words are written from the exponent's tiles, held for a
    # group of tiles (4 of 4 segments for FP8, 8 for FP4 pairs) and stored as
    # 16-byte rows (a whole group) or word by word (a group cut short by the
    # chunk's end); 21 and 40 segments give whole groups followed by a short one
    print(f"case: {dt} whole segments, mantissa raw", flush=True)
    odt = oracle.FP8_E4M3 if dt == "fp8" else oracle.FP4X2_E2M1
    seen = set()
    for k in (1, 3, 5, 6, 21, 40, 259):
        x = (W.fp8_blockscaled(1024 * k + 1, device="cuda")[0][1] if dt == "fp8"
             else W.fp4_blockscaled(1024 * k + 1, device="cuda")[0][1])
        # aligned, and one byte off 16-byte alignment (the tiles then load bytes)
        for t in (x[: 1024 * k], x[1:]):
            for cb in (4096, 262144):
                _, blob = _check_equal(oracle, odt, [t], cb)
                seen |= set(field_modes(blob.cpu().numpy(), 2, [4, 3] if dt == "fp8" else [4, 2]))
    assert (2, 0) in seen, seen


def test_empty_tensors(oracle):
    # zero-element tensors among others, and a container of one empty tensor
    # (no chunks: the chunk kernels are not launched)
    print("case: empty tensors", flush=True)
    x = W.single_bf16(1000, device="cuda")[0][1]
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    _check_equal(oracle, oracle.BF16, [e, x, e], 4096)
    _check_equal(oracle, oracle.BF16, [e], 4096)
    f = torch.empty(0, dtype=torch.float8_e4m3fn, device="cuda")
    _check_equal(oracle, oracle.FP8_E4M3, [f, W.fp8_blockscaled(3000, device="cuda")[0][1]], 4096)


@pytest.mark.parametrize("cb", [1 << 20, 12288])
def test_largest_and_odd_chunk_sizes(oracle, cb):
    # the largest chunk (1 MiB: 1024 BF16 segments, 16-bit histogram bins at
    # their limit) and a chunk of three 4 KiB pages, every dtype, 2.5 chunks
    print(f"case: every dtype at {cb}-byte chunks", flush=True)
    nb = cb * 5 // 2
    cases = [
        (oracle.BF16, [t for _, t in W.single_bf16(nb // 2, device="cuda")]),
        (oracle.FP32, [t for _, t in W.fp32_pair(nb // 4, device="cuda")]),
        (oracle.FP8_E4M3, [W.fp8_blockscaled(nb, device="cuda")[0][1]]),
        (oracle.FP4X2_E2M1, [W.fp4_blockscaled(nb, device="cuda")[0][1]]),
    ]
    for odt, tensors in cases:
        _check_equal(oracle, odt, tensors, cb)


# ------------------------------------------------------------- FP4 pairs ----
def _fp4_bytes(lo, hi):
    return (lo.to(torch.int64) | (hi.to(torch.int64) << 4)).to(torch.uint8)


def test_fp4_every_decode_path(oracle):
    print("case: FP4 pair field-mode mixes", flush=True)
    g = torch.Generator(device="cpu").manual_seed(12)
    n = 8192
    # nibble = 8 sign + 2 exponent + mantissa
    def nib(e, m, s):
        return 8 * s + 2 * e + m
    sk = lambda: torch.randint(0, 8, (n,), generator=g).clamp(max=4) // 2           # skewed 0..2
    bit = lambda: torch.randint(0, 2, (n,), generator=g)
    few = lambda: (torch.randint(0, 8, (n,), generator=g) == 0).to(torch.int64)      # mostly 0
    both = _fp4_bytes(nib(sk(), few(), bit()), nib(sk(), few(), bit()))            # E and M coded
    mraw = _fp4_bytes(nib(sk(), bit(), bit()), nib(sk(), bit(), bit()))            # E coded, M raw
    eraw = _fp4_bytes(nib(torch.randint(0, 4, (n,), generator=g), few(), bit()),
                      nib(torch.randint(0, 4, (n,), generator=g), few(), bit()))   # E raw, M coded
    const = torch.full((n,), 0x22, dtype=torch.uint8)                              # both constant
    ts = [x.cuda() for x in (both, mraw, eraw, const)]
    _, blob = _check_equal(oracle, oracle.FP4X2_E2M1, ts, 4096)
    modes = set(field_modes(blob.cpu().numpy(), 2, [4, 2]))
    assert {(2, 2), (2, 0), (0, 2), (1, 1)} <= modes, modes


def test_fp4_blockscaled(oracle):
    print("case: FP4 E2M1 pairs block-scaled 2^20 bytes", flush=True)
    x = W.fp4_blockscaled(1 << 20, device="cuda")[0][1]
    _check_equal(oracle, oracle.FP4X2_E2M1, [x], 262144)


@pytest.mark.parametrize("n", [1, 3, 15, 17, 2049, 70001])
def test_fp4_ragged_every_pattern(oracle, n):
    print(f"case: FP4 pair patterns n={n}", flush=True)
    x = (torch.arange(n, dtype=torch.int64) * 37 % 256).to(torch.uint8)
    _check_equal(oracle, oracle.FP4X2_E2M1, [x.cuda()], 4096)


# -------------------------------------------------------- single stages ----
def test_histograms_equal_bincount(oracle):
    print("case: per-chunk histograms", flush=True)
    tensors = [t for _, t in W.block_bf16("cuda", seed=2, scale=8)]
    ts = zn.setup(tensors, chunk_bytes=65536)
    h = zn.debug_histograms(ts, tensors).cpu().numpy()
    c = 0
    for t in tensors:
        e = ((to_np(t) >> 7) & 0xFF).astype(np.int64)
        for c0 in range(0, e.size, 32768):
            assert np.array_equal(h[c, 0], np.bincount(e[c0:c0 + 32768], minlength=256))
            c += 1
    assert c == h.shape[0]


def test_code_lengths_equal_oracle(oracle):
    print("case: device package-merge vs oracle", flush=True)
    rng = np.random.default_rng(11)
    hs = []
    for i in range(300):
        d = int(rng.integers(1, 257))
        h = np.zeros(256, np.int64)
        idx = rng.choice(256, d, replace=False)
        kind = i % 3
        h[idx] = (rng.integers(1, 5000, d) if kind == 0 else
                  (2.0 ** rng.uniform(0, 40, d)).astype(np.int64) + 1 if kind == 1 else
                  rng.integers(1, 3, d))
        hs.append(h)
    H = torch.from_numpy(np.stack(hs)).cuda()
    for group in (False, True):
        got = zn.debug_code_lengths(H, 256, group).cpu().numpy()
        for h, g in zip(hs, got):
            want = oracle.code_lengths(h.astype(np.uint64), group=group)
            assert np.array_equal(g, want)


# ----------------------------------------------------------- grouped setup --
def _small_model(scale=16, n_layers=2):
    return [t for _, t in W.model_bf16("cuda", seed=5, n_layers=n_layers, scale=scale)]


def test_setup_equals_oracle_and_reuses(oracle):
    print("case: grouped setup K=16 on a scaled model, reuse on a perturbed copy", flush=True)
    tensors = _small_model()
    arrs = [to_np(t) for t in tensors]
    ts = zn.setup(tensors, chunk_bytes=65536, n_groups=16)
    ots = oracle.setup(oracle.BF16, arrs, 65536, 16)
    assert ts.group_map() == ots.group_map().tolist()
    for g in range(16):
        assert ts.lengths(g) == ots.lengths(g).tolist()
    assert ts.hash == ots.hash
    assert ts.save() == ots.save()
    assert ts.cost_history() == [int(v) for v in ots.cost_history()]
    _check_equal(oracle, oracle.BF16, tensors, 65536, ts, ots)
    names = [f"t{i}" for i in range(len(tensors))]
    pert = [t for _, t in W.perturbed_model(list(zip(names, tensors)), seed=5)]
    _check_equal(oracle, oracle.BF16, pert, 65536, ts, ots)
    # a tableset reloaded from its bytes decodes the same container
    ts2 = zn.Tableset.load(ts.save())
    _, blob = gpu_compress(pert, 65536, ts)
    assert_roundtrip(ts2, blob, pert)


@pytest.mark.parametrize("dt", ["fp32", "fp8", "fp4"])
def test_setup_other_dtypes_equals_oracle(oracle, dt):
    # grouped setup (K = 4) on the exponent stream of the other dtypes: map,
    # group lengths, hash, saved bytes, cost history and containers
    print(f"case: grouped setup K=4, {dt}", flush=True)
    if dt == "fp32":
        odt, tensors = oracle.FP32, [t for _, t in W.fp32_pair(1 << 18, device="cuda")]
    elif dt == "fp8":
        odt, tensors = oracle.FP8_E4M3, [W.fp8_blockscaled(1 << 20, device="cuda")[0][1]]
    else:
        odt, tensors = oracle.FP4X2_E2M1, [W.fp4_blockscaled(1 << 20, device="cuda")[0][1]]
    arrs = [to_np(t) for t in tensors]
    ts = zn.setup(tensors, chunk_bytes=65536, n_groups=4)
    ots = oracle.setup(odt, arrs, 65536, 4)
    assert ts.group_map() == ots.group_map().tolist()
    for g in range(4):
        assert ts.lengths(g) == ots.lengths(g).tolist()
    assert ts.hash == ots.hash and ts.save() == ots.save()
    assert ts.cost_history() == [int(v) for v in ots.cost_history()]
    _check_equal(oracle, odt, tensors, 65536, ts, ots)


def test_transfer_equals_oracle(oracle):
    print("case: grouped setup K=8 on a scaled model, transferred to another architecture", flush=True)
    tensors = _small_model()
    ts = zn.setup(tensors, chunk_bytes=65536, n_groups=8)
    ots = oracle.setup(oracle.BF16, [to_np(t) for t in tensors], 65536, 8)
    other = [t for _, t in W.other_block_bf16("cuda", seed=7, scale=8)]
    other[1].view(-1)[5] = float("inf")    # a chunk no group code can code
    tr = zn.setup_transfer(ts, other)
    otr = oracle.setup_transfer(ots, [to_np(t) for t in other])
    assert tr.group_map() == otr.group_map().tolist()
    assert tr.save() == otr.save() and tr.hash == otr.hash
    assert tr.cost_history() == ts.cost_history()
    _check_equal(oracle, oracle.BF16, other, 65536, tr, otr)
    # tensors of another dtype are refused
    with pytest.raises(zn.ZnError):
        zn.setup_transfer(ts, [other[1].float()])
    # and back onto the set-up tensors themselves
    tr2 = zn.setup_transfer(ts, tensors)
    otr2 = oracle.setup_transfer(ots, [to_np(t) for t in tensors])
    assert tr2.save() == otr2.save()
    _check_equal(oracle, oracle.BF16, tensors, 65536, tr2, otr2)


def test_escape_chunk(oracle):
    print("case: escape chunk under a group tableset", flush=True)
    tensors = _small_model(n_layers=1)
    ts = zn.setup(tensors, chunk_bytes=65536, n_groups=4)
    ots = oracle.setup(oracle.BF16, [to_np(t) for t in tensors], 65536, 4)
    odd = [t.clone() for t in tensors]
    odd[0].view(-1)[17] = float("inf")
    _check_equal(oracle, oracle.BF16, odd, 65536, ts, ots)


# ------------------------------------------------------- error handling ----
def test_header_and_table_corruption_rejected(oracle):
    print("case: corrupt magic and corrupt code lengths", flush=True)
    x = W.gaussian(20000, 0.0, 0.02, torch.bfloat16, "cuda", 1, 0)
    ts, blob = gpu_compress([x], 8192)
    bad = blob.clone()
    bad[0] ^= 0xFF
    with pytest.raises(zn.ZnError) as e:
        zn.decompress(ts, bad)
    assert e.value.code == -2
    off_rec = int(np.frombuffer(blob[48:56].cpu().numpy().tobytes(), np.uint64)[0])
    bad = blob.clone()
    bad[off_rec + 8:off_rec + 8 + 128] = 0x11   # all lengths 1: not a prefix code
    with pytest.raises(zn.ZnError) as e:
        zn.decompress(ts, bad)
    assert e.value.code == -2
    # an ungrouped container decodes under any plan of the same layout ...
    same_layout = zn.setup([x], chunk_bytes=8192, n_groups=2)
    assert torch.equal(zn.decompress(same_layout, blob)[0].view(torch.int16), x.view(torch.int16))
    # ... but not under another layout
    other = zn.setup([x], chunk_bytes=16384)
    with pytest.raises(zn.ZnError) as e:
        zn.decompress(other, blob)
    assert e.value.code == -2
    # a grouped container needs the very tableset it was made with
    _, gblob = gpu_compress([x], 8192, same_layout)
    third = zn.setup([x * 3], chunk_bytes=8192, n_groups=2)
    if third.hash != same_layout.hash:
        with pytest.raises(zn.ZnError) as e:
            zn.decompress(third, gblob)
        assert e.value.code == -4
    assert oracle.decompress_status(gblob.cpu().numpy(), [x.numel()]) == -4


def test_capacity_reported():
    print("case: output buffer too small", flush=True)
    x = W.gaussian(100000, 0.0, 0.02, torch.bfloat16, "cuda", 1, 0)
    ts = zn.setup([x], chunk_bytes=65536)
    small = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(zn.ZnError) as e:
        zn.compress(ts, [x], out=small)
    assert e.value.code == -3


# ------------------------------------------------ full-size workloads ------
# Every full-size workload is compared as a whole container: the oracle
# compresses the same bits on the host (in a thread, while the GPU works) and
# the two containers must be equal byte for byte -- header, tensor table,
# directory, always-raw planes, every record and the zero tail.
def _whole_container_parity(oracle, dt, tensors, chunk_bytes, ts=None, ots=None, label=""):
    import time
    t0 = time.time()
    arrs = [to_np(t) for t in tensors]
    fut = oracle_compress_async(oracle, dt, arrs, chunk_bytes, ots)
    ts, blob = gpu_compress(tensors, chunk_bytes, ts)
    g = blob.cpu().numpy()
    print(f"  {label}: GPU container {g.size} bytes at {time.time() - t0:.0f} s", flush=True)
    assert_roundtrip(ts, blob, tensors)
    del blob
    o = fut.result()
    print(f"  {label}: oracle container {o.size} bytes at {time.time() - t0:.0f} s", flush=True)
    assert g.size == o.size and np.array_equal(g, o), first_difference(g, o)
    return ts


def test_config2_block_full_size(oracle):
    print("case: 8B-shaped BF16 block, full size, whole-container parity", flush=True)
    tensors = [t for _, t in W.block_bf16("cuda", seed=2)]
    _whole_container_parity(oracle, oracle.BF16, tensors, 262144, label="block")


def test_config3_fp32_full_size(oracle):
    print("case: FP32 regular + clean 2 x 2^27, whole-container parity", flush=True)
    tensors = [t for _, t in W.fp32_pair(1 << 27, device="cuda")]
    _whole_container_parity(oracle, oracle.FP32, tensors, 262144, label="fp32 pair")


def test_config4_fp8_full_size(oracle):
    print("case: FP8 E4M3 2^30, whole-container parity", flush=True)
    tensors = [W.fp8_blockscaled(1 << 30, device="cuda")[0][1]]
    _whole_container_parity(oracle, oracle.FP8_E4M3, tensors, 262144, label="fp8")


def test_fp4_full_size(oracle):
    print("case: FP4 E2M1 pairs 2^29 bytes, whole-container parity", flush=True)
    tensors = [W.fp4_blockscaled(1 << 29, device="cuda")[0][1]]
    _whole_container_parity(oracle, oracle.FP4X2_E2M1, tensors, 262144, label="fp4")


@pytest.mark.slow
def test_config5_full_model_grouped(oracle):
    """Full 8B-shaped model + KV cache (290 tensors, 9.65e9 BF16 values):
    the K = 16 setup on the GPU equals the oracle's on the same data, also
    with packed exponent pairs; the perturbed copy compressed with that setup
    unchanged is byte-identical to the oracle's container and round-trips
    exactly."""
    import time
    t0 = time.time()
    print("case: full model 290 tensors, K=16 setup, perturbed reuse", flush=True)
    named = W.model_bf16("cuda", seed=5)
    tensors = [t for _, t in named]
    print(f"  generated {sum(t.numel() for t in tensors)} values in {time.time() - t0:.0f} s", flush=True)
    ts = zn.setup(tensors, chunk_bytes=262144, n_groups=16)
    torch.cuda.synchronize()
    print(f"  GPU setup done at {time.time() - t0:.0f} s", flush=True)
    arrs = [to_np(t) for t in tensors]
    ots = oracle.setup(oracle.BF16, arrs, 262144, 16)
    print(f"  oracle setup done at {time.time() - t0:.0f} s", flush=True)
    assert ts.group_map() == ots.group_map().tolist()
    for g in range(16):
        assert ts.lengths(g) == ots.lengths(g).tolist()
    assert ts.hash == ots.hash and ts.save() == ots.save()
    assert ts.cost_history() == [int(v) for v in ots.cost_history()]
    # the same setup with packed exponent pairs: the grouping is the same, and
    # F, the token code lengths, the packing flags and the saved bytes (format
    # version 2) equal the oracle's
    tsp = zn.setup(tensors, chunk_bytes=262144, n_groups=16, pairs=True)
    torch.cuda.synchronize()
    otsp = oracle.setup(oracle.BF16, arrs, 262144, 16, pairs=True)
    print(f"  setups with pairs done at {time.time() - t0:.0f} s", flush=True)
    assert tsp.group_map() == ts.group_map()
    for g in range(16):
        packed, F, tl = tsp.pairs(g)
        opk, oF, otl = otsp.pairs(g)
        assert packed == opk and F == oF and tl == otl.tolist(), g
    assert tsp.hash == otsp.hash and tsp.save() == otsp.save()
    del arrs, tsp, otsp
    pert = [t for _, t in W.perturbed_model(named, seed=5)]
    del named, tensors
    _whole_container_parity(oracle, oracle.BF16, pert, 262144, ts, ots, label="perturbed model")
    print(f"  done at {time.time() - t0:.0f} s", flush=True)


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_thousands_of_small_tensors(oracle, dt):
    # a state dict of many small tensors (biases, norms, some empty): the
    # tensor table, each chunk's tensor lookup and the per-tensor raw planes
    print(f"case: {dt} 3000 small tensors", flush=True)
    rng = np.random.default_rng(17)
    sizes = [int(v) for v in rng.integers(0, 5000, 3000)]
    sizes[::97] = [0] * len(sizes[::97])
    if dt == "bf16":
        tensors = [W.gaussian(max(n, 1), 0.0, 0.02, torch.bfloat16, "cuda", i, 3)[:n] for i, n in enumerate(sizes)]
        odt = oracle.BF16
    else:
        tensors = [(torch.arange(n, dtype=torch.int64) * (i + 3) % 256).to(torch.uint8)
                   .view(torch.float8_e4m3fn).cuda() for i, n in enumerate(sizes)]
        odt = oracle.FP8_E4M3
    for cb in (4096, 16384):
        _check_equal(oracle, odt, tensors, cb)
    if dt == "bf16":
        ts = zn.setup(tensors, chunk_bytes=4096, n_groups=4)
        ots = oracle.setup(oracle.BF16, [to_np(t) for t in tensors], 4096, 4)
        assert ts.group_map() == ots.group_map().tolist() and ts.save() == ots.save()
        _check_equal(oracle, odt, tensors, 4096, ts, ots)
