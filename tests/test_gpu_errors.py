"""GPU error handling through the C ABI, against the CPU oracle.

Reconstruction must be exact or refused ("NeuralZip: Reusable Setup for Fast
Lossless Compression", Abstract; "Lossless Compression of Neural Network
Components ... in Low-Precision Formats", Abstract): a damaged container is
decoded by the GPU exactly when the oracle decodes it (then to the oracle's
output) and is otherwise refused with the oracle's status, with and without
synchronisation.  Also: plans rebuilt from a container header, saved plans
without groups, the binding's input checks, and chunks whose Huffman and raw
sections differ by at most one 16-byte step.
"""
import math

import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from lossless_float_weight_amd import zn
from tests.gpu_util import first_difference, gpu_compress, record_bounds, to_np

pytestmark = pytest.mark.gpu

NP = {zn.BF16: np.uint16, zn.FP32: np.uint32, zn.FP8_E4M3: np.uint8, zn.FP4X2_E2M1: np.uint8}
TORCH = {zn.BF16: torch.bfloat16, zn.FP32: torch.float32, zn.FP8_E4M3: torch.float8_e4m3fn,
         zn.FP4X2_E2M1: torch.uint8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zn.lib()


def _containers(oracle):
    """(name, dtype, tensors on the GPU, plan, oracle plan) of small
    multi-chunk containers of every dtype, one made with group codes."""
    out = []
    bf = [t for _, t in W.block_bf16("cuda", seed=2, scale=64)]
    out.append(("bf16", zn.BF16, bf, None, None))
    ots = oracle.setup(oracle.BF16, [to_np(t) for t in bf], 8192, 4)
    gts = zn.setup(bf, chunk_bytes=8192, n_groups=4)
    out.append(("bf16-grouped", zn.BF16, bf, gts, ots))
    out.append(("fp32", zn.FP32, [t for _, t in W.fp32_pair(12000, device="cuda")], None, None))
    out.append(("fp8", zn.FP8_E4M3, [W.fp8_blockscaled(30000, device="cuda")[0][1]], None, None))
    out.append(("fp4", zn.FP4X2_E2M1, [W.fp4_blockscaled(30000, device="cuda")[0][1]], None, None))
    return out


def _expected_status(oracle, blob_np, tensors, ots):
    """The oracle's verdict: (status, outputs).  Its argument status for a
    header naming another tensor count is a corrupt container here, where the
    plan fixes the count."""
    n = [t.numel() for t in tensors]
    st = oracle.decompress_status(blob_np, n, ots)
    if st == -1:
        st = -2
    outs = None
    if st == 0:
        outs = oracle.decompress(blob_np, n, None, ots)
    return st, outs


def _gpu_status(ts, blob_np, tensors, sync):
    dev = tensors[0].device
    blob = torch.from_numpy(blob_np.copy()).to(dev)
    outs = [torch.empty_like(t).reshape(-1) for t in tensors]
    scratch = torch.full((256,), 0xAB, dtype=torch.uint8, device=dev)
    try:
        zn.decompress(ts, blob, outs=outs, scratch=scratch, sync=sync)
        torch.cuda.synchronize()
        if not sync:
            flag = int(scratch[:4].view(torch.int32).item())
            if flag:
                return (-4 if flag & 4 else -2), None
        return 0, outs
    except zn.ZnError as e:
        return e.code, None


def _corruptions(blob, rng, n_flips):
    """Single-bit flips (anywhere, and in the header, directory, record heads,
    segment-length tables and payloads), truncations, directory entries moved
    and segment lengths off by one."""
    total = blob.size
    _, M, dirv = record_bounds(blob)
    off_dir = int(np.frombuffer(blob[40:48].tobytes(), np.uint64)[0])
    off_rec = int(np.frombuffer(blob[48:56].tobytes(), np.uint64)[0])
    cases = []
    spots = list(rng.integers(0, total, n_flips))
    spots += list(rng.integers(0, 64, 16))
    spots += list(rng.integers(off_dir, off_dir + 8 * (M + 1), 16))
    for c in rng.integers(0, M, 8):
        r0 = int(dirv[c])
        spots += [r0 + int(rng.integers(0, 8)), r0 + 8 + int(rng.integers(0, 64)),
                  int(rng.integers(r0, int(dirv[c + 1])))]
    for pos in spots:
        b = blob.copy()
        b[int(pos)] ^= np.uint8(1 << int(rng.integers(0, 8)))
        cases.append((f"flip byte {int(pos)}", b, total))
    for cut in sorted({off_rec + 16, total - 16, total - 32, (total // 2) & ~15}):
        if off_rec + 16 <= cut < total:
            cases.append((f"truncated to {cut}", blob[:cut].copy(), cut))
    for c in rng.integers(0, M, 4):
        for delta in (16, -16, 1 << 20):
            b = blob.copy()
            v = np.frombuffer(b[off_dir + 8 * int(c):off_dir + 8 * int(c) + 8].tobytes(), np.uint64)[0]
            b[off_dir + 8 * int(c):off_dir + 8 * int(c) + 8] = np.frombuffer(
                np.uint64((int(v) + delta) % (1 << 64)).tobytes(), np.uint8)
            cases.append((f"directory entry {int(c)} {delta:+d}", b, total))
    return cases


def test_damaged_containers_decode_as_the_oracle_says(oracle):
    rng = np.random.default_rng(21)
    for name, dt, tensors, ts, ots in _containers(oracle):
        print(f"case: damaged {name} containers", flush=True)
        ts, blob = gpu_compress(tensors, 8192, ts)
        g = blob.cpu().numpy()
        want = oracle.compress(dt, [to_np(t) for t in tensors], 8192, ots)
        assert np.array_equal(g, want), first_difference(g, want)
        for i, (what, bad, _) in enumerate(_corruptions(g, rng, 40)):
            est, eouts = _expected_status(oracle, bad, tensors, ots)
            for sync in ((True, False) if i % 4 == 0 else (True,)):
                st, outs = _gpu_status(ts, bad, tensors, sync)
                assert st == est, f"{name} {what} sync={sync}: GPU {st}, oracle {est}"
                if st == 0:
                    for o, e in zip(outs, eouts):
                        assert np.array_equal(W.bits(o).cpu().numpy(), e), f"{name} {what}: output"


def test_segment_lengths_off_by_one(oracle):
    # each Huffman segment's stored bit length moved by one (its neighbour's
    # the other way, so the payload size still matches): refused by both
    print("case: segment bit lengths off by one", flush=True)
    x = W.single_bf16(60000, device="cuda")[0][1]
    ts, blob = gpu_compress([x], 16384)
    g = blob.cpu().numpy()
    _, M, dirv = record_bounds(g)
    rng = np.random.default_rng(3)
    for c in range(M):
        r0 = int(dirv[c])
        mode, nseg = g[r0], int(np.frombuffer(g[r0 + 2:r0 + 4].tobytes(), np.uint16)[0])
        if mode != 2 or nseg < 2:
            continue
        j = int(rng.integers(0, nseg - 1))
        at = r0 + 8 + 128 + 2 * j
        b = g.copy()
        seg = np.frombuffer(b[at:at + 4].tobytes(), np.uint16).astype(np.int64)
        b[at:at + 4] = np.frombuffer(np.array([seg[0] + 1, seg[1] - 1], np.uint16).tobytes(), np.uint8)
        est, _ = _expected_status(oracle, b, [x], None)
        for sync in (True, False):
            st, _ = _gpu_status(ts, b, [x], sync)
            assert st == est == -2, (c, j, st, est)


def test_group_code_in_an_ungrouped_container_is_refused(oracle):
    # a record naming a group code inside a container made without groups,
    # decoded under a plan that has groups: the oracle refuses it, so must
    # the GPU
    print("case: group mode in an ungrouped container", flush=True)
    x = W.single_bf16(40000, device="cuda")[0][1]
    plain = zn.setup([x], chunk_bytes=16384)
    grouped = zn.setup([x], chunk_bytes=16384, n_groups=2)
    _, blob = gpu_compress([x], 16384, plain)
    g = blob.cpu().numpy()
    _, M, dirv = record_bounds(g)
    r0 = int(dirv[0])
    assert g[r0] == 2
    b = g.copy()
    b[r0] = 3          # GROUP, group 0
    assert oracle.decompress_status(b, [x.numel()]) == -2
    st, _ = _gpu_status(grouped, b, [x], True)
    assert st == -2


def test_huff_raw_boundary_chunks(oracle):
    # Chunks whose own Huffman section and raw section differ by at most one
    # 16-byte step.  The encoder may skip the code build when the entropy
    # bound (n*H bits, lowered by a small margin) already gives a Huffman
    # section no smaller than the raw one; chunks are picked by (Huffman -
    # raw, bound - raw) in bytes: the bound exactly at the raw size with the
    # code one step over it, a tie (goes to raw) with the bound one step
    # under, and the code one step under raw.  The choices must be the
    # oracle's exactly.
    print("case: chunks at the Huffman / raw boundary", flush=True)
    rng = np.random.default_rng(5)
    n, nseg = 4096, 8
    a16 = lambda v: (v + 15) & ~15   # noqa: E731
    raw = a16(8) + a16(n)
    want = {(16, 0): [], (16, -16): [], (0, -16): [], (0, -32): [], (-16, -32): []}
    for _ in range(20000):
        if all(len(v) >= 8 for v in want.values()):
            break
        alpha = rng.uniform(0.5, 0.7)
        p = np.exp(-alpha * rng.standard_normal(256))
        e = rng.choice(256, n, p=p / p.sum())
        h = np.bincount(e, minlength=256).astype(np.uint64)
        bits = int((h * oracle.code_lengths(h).astype(np.uint64)).sum())
        huff = a16(8 + 128 + 2 * nseg) + a16(4 * ((bits + 31) // 32))
        H = -sum(int(c) / n * math.log2(int(c) / n) for c in h if c)
        lb = int(n * H * (1 - 1e-9) - 64)
        bound = a16(8 + 128 + 2 * nseg) + a16(4 * ((lb + 31) // 32))
        key = (huff - raw, bound - raw)
        if key in want and len(want[key]) < 8:
            want[key].append(e)
    assert all(len(v) == 8 for v in want.values()), {k: len(v) for k, v in want.items()}
    ex = np.concatenate([e for v in want.values() for e in v]).astype(np.uint16)
    sf = rng.integers(0, 256, ex.size).astype(np.uint16)
    w = ((sf & 0x80) << 8) | (ex << 7) | (sf & 0x7F)
    x = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    ts, blob = gpu_compress([x], 2 * n)
    g = blob.cpu().numpy()
    o = oracle.compress(oracle.BF16, [w], 2 * n)
    assert np.array_equal(g, o), first_difference(g, o)
    _, M, dirv = record_bounds(g)
    modes = [int(g[int(dirv[c])]) for c in range(M)]
    assert modes == [0] * 32 + [2] * 8, modes
    out = zn.decompress(ts, blob)[0]
    assert torch.equal(W.bits(out).cpu(), torch.from_numpy(w.view(np.int16)).view(torch.uint16))


def test_plan_from_container_and_header_info(oracle):
    print("case: plan rebuilt from a container header", flush=True)
    tensors = [t for _, t in W.block_bf16("cuda", seed=2, scale=32)]
    ts, blob = gpu_compress(tensors, 16384)
    info = zn.header_info(blob)
    assert info == oracle.header(blob.cpu().numpy())
    plan = zn.plan_from_container(blob)
    a, b = plan.info(), ts.info()
    for k in ("dtype", "n_tensors", "n_elems", "chunk_bytes", "n_chunks", "n_groups", "hash"):
        assert a[k] == b[k], k
    outs = zn.decompress(plan, blob)
    for x, y in zip(tensors, outs):
        assert torch.equal(W.bits(x).reshape(-1), W.bits(y))
    # a damaged header or tensor table is refused
    for pos in (0, 6, 12, 24, 40, 48, 64, 72):
        bad = blob.clone()
        bad[pos] ^= 0x10
        with pytest.raises(zn.ZnError) as e:
            zn.plan_from_container(bad)
        assert e.value.code == -2, pos
    # a container made with group codes needs its own tableset
    gts = zn.setup(tensors, chunk_bytes=16384, n_groups=2)
    _, gblob = gpu_compress(tensors, 16384, gts)
    assert zn.header_info(gblob)["tableset_hash"] == gts.hash
    with pytest.raises(zn.ZnError) as e:
        zn.plan_from_container(gblob)
    assert e.value.code == -4


@pytest.mark.parametrize("dt", [zn.BF16, zn.FP8_E4M3])
def test_plan_without_groups_saves_and_reloads(oracle, dt):
    print(f"case: plan without groups saved and reloaded, dtype {dt}", flush=True)
    x = (W.single_bf16(50000, device="cuda")[0][1] if dt == zn.BF16
         else W.fp8_blockscaled(50000, device="cuda")[0][1])
    ts = zn.setup([x], chunk_bytes=8192)
    saved = ts.save()
    odt = oracle.BF16 if dt == zn.BF16 else oracle.FP8_E4M3
    assert saved == oracle.setup(odt, [to_np(x)], 8192, 0).save()
    back = zn.Tableset.load(saved)
    assert back.save() == saved and back.hash == ts.hash
    _, blob = gpu_compress([x], 8192, ts)
    y = zn.decompress(back, blob)[0]
    assert torch.equal(W.bits(x), W.bits(y))


def test_binding_refuses_mismatched_tensors():
    print("case: mismatched tensors refused before any launch", flush=True)
    x = W.single_bf16(10000, device="cuda")[0][1]
    ts = zn.setup([x], chunk_bytes=8192)
    with pytest.raises(zn.ZnError):
        zn.compress(ts, [x, x])                                      # count
    with pytest.raises(zn.ZnError):
        zn.compress(ts, [x[:9999]])                                  # size
    with pytest.raises(zn.ZnError):
        zn.compress(ts, [x.float()])                                 # dtype
    with pytest.raises(zn.ZnError):
        zn.compress(ts, [x.cpu()])                                   # device
    m = x[:10000 - 16].reshape(-1, 16)[:, :8]
    ts2 = zn.setup(n_elems=[m.numel()], dtype=zn.BF16, chunk_bytes=8192)
    with pytest.raises(zn.ZnError):
        zn.compress(ts2, [m])                                        # strided view
    blob = zn.compress(ts, [x])
    with pytest.raises(zn.ZnError):
        zn.decompress(ts, blob, outs=[torch.empty(9999, dtype=torch.bfloat16, device="cuda")])
    with pytest.raises(zn.ZnError):
        zn.decompress(ts, blob, outs=[torch.empty(10000, dtype=torch.float16, device="cuda")])


def test_two_streams_overlapping_calls():
    # two plans on two streams (default priority): both compressions run at
    # once, each decompression follows its compression on the other stream by
    # an event; containers equal the ones made alone, outputs equal inputs
    print("case: overlapping calls on two streams", flush=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xa = [t for _, t in W.block_bf16("cuda", seed=2, scale=8)]
    xb = [W.fp8_blockscaled(1 << 20, device="cuda")[0][1]]
    tsa = zn.setup(xa, chunk_bytes=262144)
    tsb = zn.setup(xb, chunk_bytes=65536)
    ref_a = zn.compress(tsa, xa).cpu()
    ref_b = zn.compress(tsb, xb).cpu()
    outa = torch.empty(zn.compress_bound(tsa), dtype=torch.uint8, device="cuda")
    outb = torch.empty(zn.compress_bound(tsb), dtype=torch.uint8, device="cuda")
    ya = [torch.empty_like(t) for t in xa]
    yb = [torch.empty_like(t) for t in xb]
    torch.cuda.synchronize()
    for rep in range(3):
        outa.fill_(0xEE)
        outb.fill_(0xEE)
        torch.cuda.synchronize()
        zn.compress(tsa, xa, out=outa, sync=False, stream=s1)
        zn.compress(tsb, xb, out=outb, sync=False, stream=s2)
        ea, eb = torch.cuda.Event(), torch.cuda.Event()
        ea.record(s1)
        eb.record(s2)
        s2.wait_event(ea)
        s1.wait_event(eb)
        zn.decompress(tsa, outa[: ref_a.numel()], outs=ya, sync=False, stream=s2)
        zn.decompress(tsb, outb[: ref_b.numel()], outs=yb, sync=False, stream=s1)
        torch.cuda.synchronize()
        assert torch.equal(outa[: ref_a.numel()].cpu(), ref_a), rep
        assert torch.equal(outb[: ref_b.numel()].cpu(), ref_b), rep
        for x, y in zip(xa + xb, ya + yb):
            assert torch.equal(W.bits(x).reshape(-1), W.bits(y).reshape(-1)), rep
