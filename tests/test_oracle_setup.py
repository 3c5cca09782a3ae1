"""Oracle pins for the NeuralZip-style reusable setup.

"NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract: chunks
with similar exponent distributions are grouped and share Huffman codes; a
setup picks these before later encodings, each of which still reads the
current values; reconstruction is exact; the setup stays usable as weights
evolve, with similar ratios.  Pins:
  * one group reproduces the code of the pooled histogram (K = 1);
  * the Lloyd objective never increases from round to round;
  * a shared table never beats the chunk's own optimal table;
  * round trip on the set-up tensors and on a perturbed copy;
  * the whole tableset (map and tables) equals an independent restatement of
    the grouping on a small case.
"""
import numpy as np
import pytest
import torch

from lossless_float_weight_amd import workloads as W
from tests import ref_tiny


def _model(scale=16, n_layers=2, seed=5):
    ts = W.model_bf16("cpu", seed=seed, n_layers=n_layers, scale=scale, kv_tokens=32768)
    return ts


def _np(tensors):
    return [W.bits(t).numpy().ravel() for _, t in tensors]


def test_single_group_is_pooled_code(oracle):
    arrs = _np(_model())
    ts = oracle.setup(oracle.BF16, arrs, 65536, 1)
    pooled = np.zeros(256, np.uint64)
    for a in arrs:
        pooled += np.bincount(((a >> 7) & 0xFF).astype(np.int64), minlength=256).astype(np.uint64)
    assert ts.lengths(0).tolist() == oracle.code_lengths(pooled, group=True).tolist()
    assert np.all(ts.group_map() == 0)


def test_cost_non_increasing(oracle):
    arrs = _np(_model())
    ts = oracle.setup(oracle.BF16, arrs, 65536, 16)
    cost = ts.cost_history()
    assert np.all(cost[1:] <= cost[:-1])
    assert cost[-1] < cost[0] or cost[0] == cost[-1]


def test_group_payload_not_below_own_code(oracle):
    arrs = _np(_model())
    ts = oracle.setup(oracle.BF16, arrs, 65536, 8)
    _, st_g = oracle.compress(oracle.BF16, arrs, 65536, ts, with_stats=True)
    _, st_h = oracle.compress(oracle.BF16, arrs, 65536, None, with_stats=True)
    assert st_g["payload_bits"][0] >= st_h["payload_bits"][0]
    assert st_g["mode_count"][0][oracle.GROUP] > 0


def test_roundtrip_original_and_perturbed(oracle):
    model = _model()
    arrs = _np(model)
    ts = oracle.setup(oracle.BF16, arrs, 65536, 16)
    blob, st = oracle.compress(oracle.BF16, arrs, 65536, ts, with_stats=True)
    for a, b in zip(arrs, oracle.decompress(blob, [a.size for a in arrs], ts=ts)):
        assert np.array_equal(a, b)
    pert = _np(W.perturbed_model(model, seed=5))
    blob_p, st_p = oracle.compress(oracle.BF16, pert, 65536, ts, with_stats=True)
    for a, b in zip(pert, oracle.decompress(blob_p, [a.size for a in pert], ts=ts)):
        assert np.array_equal(a, b)
    # similar ratio after the perturbation (no number on the page: reported band)
    assert abs(blob_p.size - blob.size) / blob.size < 0.01
    # decoding without the tableset is refused, and so is another tableset
    assert oracle.decompress_status(blob, [a.size for a in arrs]) == -4
    other = oracle.setup(oracle.BF16, arrs, 65536, 3)
    assert oracle.decompress_status(blob, [a.size for a in arrs], other) == -4


def test_escape_chunk_uses_own_table(oracle):
    base = _np(_model(n_layers=1))
    ts = oracle.setup(oracle.BF16, base, 65536, 4)
    odd = [a.copy() for a in base]
    odd[0][17] = 0x7F80          # +inf: exponent 255, absent from every table
    blob, st = oracle.compress(oracle.BF16, odd, 65536, ts, with_stats=True)
    assert st["escapes"] == 1
    for a, b in zip(odd, oracle.decompress(blob, [a.size for a in odd], ts=ts)):
        assert np.array_equal(a, b)


def test_tableset_save_load(oracle):
    arrs = _np(_model(n_layers=1))
    ts = oracle.setup(oracle.BF16, arrs, 65536, 5)
    data = ts.save()
    ts2 = oracle.Tableset.load(data)
    assert ts2.hash == ts.hash
    assert ts2.group_map().tolist() == ts.group_map().tolist()
    blob = oracle.compress(oracle.BF16, arrs, 65536, ts)
    for a, b in zip(arrs, oracle.decompress(blob, [a.size for a in arrs], ts=ts2)):
        assert np.array_equal(a, b)
    bad = bytearray(data)
    bad[-1] = 200                # group id out of range
    with pytest.raises(Exception):
        oracle.Tableset.load(bytes(bad))


def _ref_setup(hists, sizes, K, rounds=8, A=256):
    """Independent restatement of the grouping (Python integers)."""
    M = len(hists)
    keys = sorted(((sum(s * h[s] for s in range(A)) << 16) // sizes[c], c) for c, h in enumerate(hists))
    grp = [0] * M
    for g in range(K):
        for i in range(M * g // K, M * (g + 1) // K):
            grp[keys[i][1]] = g

    def tables(grp):
        out = []
        for g in range(K):
            H = [0] * A
            for c in range(M):
                if grp[c] == g:
                    H = [a + b for a, b in zip(H, hists[c])]
            out.append(ref_tiny.group_lengths(H))
        return out

    def cost(h, ln):
        if any(h[s] and not ln[s] for s in range(A)):
            return None
        return sum(h[s] * ln[s] for s in range(A))

    for _ in range(rounds):
        tab = tables(grp)
        new = []
        for c in range(M):
            best, bg = None, grp[c]
            for g in range(K):
                x = cost(hists[c], tab[g])
                if x is not None and (best is None or x < best):
                    best, bg = x, g
            new.append(bg)
        grp = new
    return grp, tables(grp)


def test_grouping_matches_independent_restatement(oracle):
    arrs = _np(_model(scale=32, n_layers=2))
    cb = 16384
    ce = cb // 2
    hists, sizes = [], []
    for a in arrs:
        e = ((a >> 7) & 0xFF).astype(np.int64)
        for c0 in range(0, a.size, ce):
            hists.append([int(v) for v in np.bincount(e[c0:c0 + ce], minlength=256)])
            sizes.append(min(ce, a.size - c0))
    K = 6
    ts = oracle.setup(oracle.BF16, arrs, cb, K)
    grp, tab = _ref_setup(hists, sizes, K)
    assert ts.group_map().tolist() == grp
    for g in range(K):
        assert ts.lengths(g).tolist() == tab[g]


# ------------------------------------------------------------- tableset hash
def _fnv_vectors():
    import ast
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "fnv1a64_vectors.txt")
    out = []
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            lit, hx = line.rstrip("\n").split("\t")
            out.append((ast.literal_eval(lit), int(hx, 16)))
    return out


def test_fnv1a64_restatement_matches_published_vectors():
    vecs = _fnv_vectors()
    assert len(vecs) >= 3
    for data, want in vecs:
        assert ref_tiny.fnv1a64(data) == want, data


@pytest.mark.parametrize("K", [0, 1, 4])
def test_tableset_hash_is_fnv1a64_of_saved_bytes(oracle, K):
    # the hash a grouped container records is FNV-1a-64 over the saved
    # tableset; the restatement above is pinned to the published vectors
    arrs = _np(_model(n_layers=1))
    ts = oracle.setup(oracle.BF16, arrs, 65536, K)
    assert ts.hash == ref_tiny.fnv1a64(ts.save())
    blob = oracle.compress(oracle.BF16, arrs, 65536, ts)
    h = oracle.header(blob)
    assert h["tableset_hash"] == (ref_tiny.fnv1a64(ts.save()) if K else 0)


def test_transferred_tableset_hash_is_fnv1a64(oracle):
    arrs = _np(_model(n_layers=1))
    ts = oracle.setup(oracle.BF16, arrs, 65536, 4)
    other = [W.bits(t).numpy().ravel() for _, t in W.other_block_bf16("cpu", seed=7, scale=16)]
    tr = oracle.setup_transfer(ts, other)
    assert tr.hash == ref_tiny.fnv1a64(tr.save()) and tr.hash != ts.hash


def test_plan_without_groups_saves_and_loads(oracle):
    # a plan with no groups stores its chunk map as zero bytes and loads back
    arrs = _np(_model(n_layers=1))
    ts = oracle.setup(oracle.BF16, arrs, 65536, 0)
    saved = ts.save()
    assert ts.n_groups == 0 and ts.group_map().size > 0 and not np.any(ts.group_map())
    back = oracle.Tableset.load(saved)
    assert back.save() == saved and back.hash == ts.hash
    # a non-zero map byte in such a plan is corrupt
    bad = bytearray(saved)
    bad[-1] = 1
    with pytest.raises(oracle.OracleError):
        oracle.Tableset.load(bytes(bad))
