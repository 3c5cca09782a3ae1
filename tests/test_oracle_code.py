"""Oracle pins for the code construction (order-0 Huffman, length-limited).

THEORY-599 (nucleation note on ZipNN) describes an order-0 Huffman coder of
the exponent and, under "implied entropy", a Huffman code length within one
bit of the order-0 entropy.  The oracle builds optimal prefix codes limited to
11 bits by package-merge.  Pins, none of which re-runs the oracle's own
formula:
  * Kraft equality and the length limit (Kraft-McMillan, textbook);
  * optimality against brute force over every admissible length vector;
  * equality with the cost of Huffman's algorithm whenever the limit is slack;
  * H <= mean length < H + 1 on exponent-like histograms;
  * a more frequent symbol never gets a longer code;
  * the exact length vector against an independent coin-collector
    implementation (tests/ref_tiny.py) under the same tie rule;
  * canonical codes: RFC 1951 section 3.2.2 worked example, prefix-freeness.
"""
import math
import os

import numpy as np
import pytest

from tests import ref_tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cost(h, ln):
    return int(sum(int(a) * int(b) for a, b in zip(h, ln)))


def _kraft_sum(ln, L=11):
    return sum(1 << (L - int(l)) for l in ln if l)


def _random_hists(rng, n):
    for _ in range(n):
        A = int(rng.choice([8, 16, 256]))
        d = int(rng.integers(2, A + 1))
        h = np.zeros(A, np.uint64)
        idx = rng.choice(A, d, replace=False)
        kind = rng.integers(0, 3)
        if kind == 0:
            h[idx] = rng.integers(1, 1000, d)
        elif kind == 1:  # geometric: forces deep codes
            h[idx] = np.maximum(1, (2.0 ** rng.uniform(0, 30, d))).astype(np.uint64)
        else:  # many ties
            h[idx] = rng.integers(1, 4, d)
        yield h


def test_kraft_equality_and_limit(oracle):
    rng = np.random.default_rng(1)
    for h in _random_hists(rng, 300):
        ln = oracle.code_lengths(h)
        assert ln.max() <= 11
        assert np.all((ln > 0) == (h > 0))
        assert _kraft_sum(ln) == 1 << 11


@pytest.mark.parametrize("d", [2, 3, 4, 5, 6, 7])
def test_optimal_against_brute_force(oracle, d):
    rng = np.random.default_rng(100 + d)
    for trial in range(12):
        w = rng.integers(1, 60, d) if trial % 2 else (2 ** rng.integers(0, 12, d))
        h = np.zeros(16, np.uint64)
        h[rng.choice(16, d, replace=False)] = w
        for L in range(max(1, math.ceil(math.log2(d))), 8):
            ln = oracle.code_lengths(h, max_len=L)
            assert ln.max() <= L
            assert _cost(h, ln) == ref_tiny.brute_force_min_cost([int(v) for v in h if v], L)


def test_equals_huffman_when_limit_slack(oracle):
    rng = np.random.default_rng(2)
    checked = 0
    for h in _random_hists(rng, 400):
        if ref_tiny.huffman_depth([int(v) for v in h]) <= 11:
            assert _cost(h, oracle.code_lengths(h)) == ref_tiny.huffman_cost([int(v) for v in h])
            checked += 1
    assert checked > 100


def test_limit_binds_and_costs_little(oracle):
    # a geometric histogram whose Huffman tree is 20 deep
    h = np.array([2 ** i for i in range(21)], np.uint64)
    ln = oracle.code_lengths(h, max_len=11)
    assert ln.max() == 11 and _kraft_sum(ln) == 1 << 11
    assert _cost(h, ln) >= ref_tiny.huffman_cost([int(v) for v in h])


def test_within_one_bit_of_entropy(oracle):
    rng = np.random.default_rng(3)
    for std in [0.005, 0.02, 0.05, 1.0]:
        x = (rng.standard_normal(131072) * std).astype(np.float32)
        e = ((x.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
        h = np.bincount(e, minlength=256).astype(np.uint64)
        ln = oracle.code_lengths(h)
        mean = _cost(h, ln) / h.sum()
        H = ref_tiny.entropy_bits([int(v) for v in h])
        assert H <= mean < H + 1


def test_frequent_symbol_never_longer(oracle):
    rng = np.random.default_rng(4)
    for h in _random_hists(rng, 200):
        ln = oracle.code_lengths(h)
        nz = np.nonzero(h)[0]
        for a in nz:
            for b in nz:
                if h[a] > h[b]:
                    assert ln[a] <= ln[b]


def test_exact_vector_matches_independent_package_merge(oracle):
    rng = np.random.default_rng(5)
    for h in _random_hists(rng, 150):
        for L in (8, 9, 11):
            if np.count_nonzero(h) > (1 << L):
                continue
            assert oracle.code_lengths(h, max_len=L).tolist() == ref_tiny.package_merge(
                [int(v) for v in h], L)


def test_degenerate_histograms(oracle):
    assert oracle.code_lengths(np.zeros(256, np.uint64)).sum() == 0
    one = np.zeros(256, np.uint64)
    one[7] = 5
    assert oracle.code_lengths(one).sum() == 0                # constant stream: no code
    g = oracle.code_lengths(one, group=True)                  # group table: complete code
    assert g[7] == 1 and g[0] == 1 and g.sum() == 2
    two = np.zeros(8, np.uint64)
    two[[2, 5]] = [1, 1000]
    assert oracle.code_lengths(two)[[2, 5]].tolist() == [1, 1]
    full = np.ones(256, np.uint64)
    assert np.all(oracle.code_lengths(full) == 8)             # uniform 256 -> 8 bits each


def test_canonical_rfc1951_example(oracle):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "rfc1951_canonical.txt"))
            if l.strip() and not l.startswith("#")]
    lens = np.array([int(r[1]) for r in rows], np.uint8)
    codes = oracle.canonical_codes(lens, max_len=4)
    for r, c in zip(rows, codes):
        assert format(int(c), "0{}b".format(int(r[1]))) == r[2]
    assert ref_tiny.canonical([int(r[1]) for r in rows]) == [int(r[2], 2) for r in rows]


def test_canonical_prefix_free_and_ordered(oracle):
    rng = np.random.default_rng(6)
    for h in _random_hists(rng, 100):
        ln = oracle.code_lengths(h)
        codes = oracle.canonical_codes(ln)
        words = [format(int(c), "0{}b".format(int(l))) for c, l in zip(codes, ln) if l]
        for a in words:
            for b in words:
                assert a == b or not b.startswith(a)
        # within one length, codes are consecutive and increase with the symbol
        for l in set(ln.tolist()) - {0}:
            cs = [int(codes[s]) for s in range(len(ln)) if ln[s] == l]
            assert cs == list(range(cs[0], cs[0] + len(cs)))


def test_length_limit_costs_little_on_weight_exponents(oracle):
    # exponents of N(0, sigma) BF16 chunks: the 11-bit limit binds (unlimited
    # Huffman trees are 14-16 deep) but adds under 0.2% to the coded bits
    import torch
    for sigma in (0.008, 0.02, 0.03):
        g = torch.Generator().manual_seed(int(sigma * 1e4))
        x = (torch.randn(131072, dtype=torch.float64, generator=g) * sigma).to(torch.bfloat16)
        e = ((x.view(torch.int16).numpy().astype(np.uint16) >> 7) & 0xFF).astype(np.int64)
        h = np.bincount(e, minlength=256).astype(np.uint64)
        ln = oracle.code_lengths(h, max_len=11)
        free = ref_tiny.huffman_cost([int(v) for v in h if v])
        assert ln.max() <= 11 and ref_tiny.huffman_depth([int(v) for v in h if v]) > 11
        assert free <= _cost(h, ln) <= free * 1.002
