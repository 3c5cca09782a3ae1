"""Independent pure-Python restatement of the codec, for tiny inputs only.

Test infrastructure: written separately from both the C oracle and the GPU
library (different data structures, no shared code), so that a slip in either
shows up as a disagreement on small cases.  Python integers, one bit at a time.

Textbook pieces restated here:
  * Huffman's algorithm with a binary heap (optimal unlimited code cost);
  * brute-force search of all length vectors obeying the Kraft-McMillan
    inequality (optimal length-limited cost);
  * package-merge as a coin collector whose items carry explicit symbol
    multisets (Larmore and Hirschberg, 1990);
  * canonical codes and LSB-first packing (RFC 1951 sections 3.1.1, 3.2.2).
"""
from __future__ import annotations

import heapq
import itertools
import math
import struct
from collections import Counter

MAX_LEN = 11
RAW, CONST, HUFF, GROUP = 0, 1, 2, 3
ESIZE = {0: 2, 1: 4, 2: 1, 3: 1}
NCODED = {0: 1, 1: 4, 2: 2, 3: 2}
SEG = {0: 512, 1: 256, 2: 1024, 3: 1024}


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit (Fowler, Noll and Vo): start from the offset basis, then
    per byte XOR it into the low bits and multiply by the 64-bit FNV prime
    2^40 + 2^8 + 0xB3, modulo 2^64."""
    prime = (1 << 40) + (1 << 8) + 0xB3
    h = 0xCBF29CE484222325
    for b in data:
        h = ((h ^ b) * prime) % (1 << 64)
    return h


def kbits(dt, p):
    if dt == 2:
        return 4 if p == 0 else 3
    if dt == 3:
        return 4 if p == 0 else 2
    return 8


# ------------------------------------------------------------ code lengths --
def huffman_cost(weights):
    """Total coded bits of Huffman's algorithm (sum of all merge weights)."""
    w = [x for x in weights if x > 0]
    if len(w) < 2:
        return 0
    heapq.heapify(w)
    cost = 0
    while len(w) > 1:
        a, b = heapq.heappop(w), heapq.heappop(w)
        cost += a + b
        heapq.heappush(w, a + b)
    return cost


def huffman_depth(weights):
    """Longest code length of one Huffman tree (ties broken by insertion)."""
    items = [(x, i, 0) for i, x in enumerate(w for w in weights if w > 0)]
    if len(items) < 2:
        return 0
    heapq.heapify(items)
    nxt = len(items)
    while len(items) > 1:
        a, b = heapq.heappop(items), heapq.heappop(items)
        heapq.heappush(items, (a[0] + b[0], nxt, max(a[2], b[2]) + 1))
        nxt += 1
    return items[0][2]


def brute_force_min_cost(weights, max_len):
    """min sum(w*l) over l in {1..max_len}^d with sum 2^-l <= 1."""
    w = [x for x in weights if x > 0]
    d = len(w)
    if d < 2:
        return 0
    best = None
    for ls in itertools.product(range(1, max_len + 1), repeat=d):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            c = sum(a * b for a, b in zip(w, ls))
            best = c if best is None or c < best else best
    return best


def package_merge(hist, max_len=MAX_LEN):
    """Length vector under the codec's tie rule; zeros when < 2 symbols occur."""
    leaves = sorted((w, s) for s, w in enumerate(hist) if w > 0)
    d = len(leaves)
    out = [0] * len(hist)
    if d < 2:
        return out
    leaf_items = [(w, 0, Counter({s: 1})) for w, s in leaves]
    cur = list(leaf_items)
    for _ in range(max_len - 1):
        packages = [(cur[2 * k][0] + cur[2 * k + 1][0], 1, cur[2 * k][2] + cur[2 * k + 1][2])
                    for k in range(len(cur) // 2)]
        # stable sort: leaves (kind 0) before packages at equal weight,
        # each kind keeps its own order
        cur = sorted(leaf_items + packages, key=lambda it: (it[0], it[1]))
    total = Counter()
    for it in cur[:2 * d - 2]:
        total += it[2]
    for s in range(len(hist)):
        out[s] = total[s]
    return out


def group_lengths(hist, max_len=MAX_LEN):
    h = list(hist)
    present = [s for s, w in enumerate(h) if w > 0]
    if not present:
        return [0] * len(h)
    if len(present) == 1:
        partner = 0 if present[0] != 0 else 1
        # a zero-weight leaf: give it a tiny marker and solve by hand
        lens = [0] * len(h)
        lens[present[0]] = 1
        lens[partner] = 1
        return lens
    return package_merge(h, max_len)


def canonical(lengths):
    """RFC 1951 section 3.2.2 code values."""
    maxl = max(lengths) if lengths else 0
    bl = [0] * (maxl + 2)
    for l in lengths:
        if l:
            bl[l] += 1
    code, nxt = 0, [0] * (maxl + 2)
    for bits in range(1, maxl + 1):
        code = (code + bl[bits - 1]) << 1
        nxt[bits] = code
    out = []
    for l in lengths:
        if l:
            out.append(nxt[l])
            nxt[l] += 1
        else:
            out.append(0)
    return out


def entropy_bits(hist):
    n = sum(hist)
    return -sum(w / n * math.log2(w / n) for w in hist if w) if n else 0.0


# ----------------------------------------------------------------- fields --
def split(dt, w):
    if dt == 0:
        return [(w >> 7) & 0xFF], ((w >> 8) & 0x80) | (w & 0x7F)
    if dt == 1:
        return [(w >> 23) & 0xFF, ((w >> 24) & 0x80) | ((w >> 16) & 0x7F), (w >> 8) & 0xFF,
                w & 0xFF], 0
    if dt == 3:
        # two FP4 E2M1 values, the first in the low nibble; a nibble reads
        # 8*sign + 2*exponent + mantissa
        lo, hi = w % 16, w // 16
        e = [(v // 2) % 4 for v in (lo, hi)]
        m = [v % 2 for v in (lo, hi)]
        sg = [v // 8 for v in (lo, hi)]
        return [e[0] + 4 * e[1], m[0] + 2 * m[1]], sg[0] + 2 * sg[1]
    return [(w >> 3) & 0xF, w & 7], w >> 7


def merge(dt, syms, raw):
    if dt == 0:
        return ((raw & 0x80) << 8) | (syms[0] << 7) | (raw & 0x7F)
    if dt == 1:
        return ((syms[1] & 0x80) << 24) | (syms[0] << 23) | ((syms[1] & 0x7F) << 16) | \
            (syms[2] << 8) | syms[3]
    if dt == 3:
        nib = [8 * (raw % 2) + 2 * (syms[0] % 4) + syms[1] % 2,
               8 * (raw // 2) + 2 * (syms[0] // 4) + syms[1] // 2]
        return nib[0] + 16 * nib[1]
    return (raw << 7) | (syms[0] << 3) | syms[1]


# ------------------------------------------------------------------- bits --
class Bits:
    def __init__(self):
        self.v = 0
        self.n = 0

    def put(self, bit):
        self.v |= (bit & 1) << self.n
        self.n += 1

    def code(self, c, l):
        for i in range(l - 1, -1, -1):
            self.put(c >> i)

    def value(self, v, k):
        for i in range(k):
            self.put(v >> i)

    def tobytes(self, nbytes):
        return self.v.to_bytes(nbytes, "little")


def a16(x):
    return (x + 15) & ~15


STRIP = 32


def segment_order(n, nseg, j):
    """Symbol indices of segment j: strips j, j + nseg, ... of 32 symbols."""
    out = []
    q = j
    while q * STRIP < n:
        out.extend(range(q * STRIP, min(n, q * STRIP + STRIP)))
        q += nseg
    return out


TANS = 4
TANS_LOG = 11
TANS_STEP = 1283


def section(mode, k, n, nseg, bits, d=0):
    head = 8 + ((1 << k) // 2 if mode == HUFF else 0) + (2 * nseg if mode in (HUFF, GROUP) else 0)
    if mode == TANS:
        head = 8 + (1 << k) // 8 + 2 * d + 2 * nseg
    pay = 4 * ((bits + 31) // 32) if mode in (HUFF, GROUP, TANS) else ((n * k + 7) // 8 if mode == RAW else 0)
    return a16(head), pay


# ----------------------------------------------------------------- tANS ----
# Restated from the description of tabled asymmetric numeral systems (Duda):
# a table of L = 2^11 states in which symbol s owns q[s] states; decoding a
# state yields its symbol and, with the state's rank among that symbol's
# states, the next state after reading a few bits; encoding runs backwards.
def tans_normalize(h):
    """Counts q with sum L, q >= 1 for present symbols (largest remainders
    fill a shortfall, ties to the smaller symbol; an excess is taken one at a
    time from the largest count, ties to the smaller symbol)."""
    L = 1 << TANS_LOG
    n = sum(h)
    q = [0] * len(h)
    for s, c in enumerate(h):
        if c:
            q[s] = max(1, c * L // n)
    short = L - sum(q)
    if short > 0:
        ranked = sorted((s for s, c in enumerate(h) if c), key=lambda s: (-((h[s] * L) % n), s))
        for s in ranked[:short]:
            q[s] += 1
    heap = [(-v, s) for s, v in enumerate(q) if v > 1]
    heapq.heapify(heap)
    while sum(q) > L:
        v, s = heapq.heappop(heap)
        q[s] -= 1
        if q[s] > 1:
            heapq.heappush(heap, (-q[s], s))
    return q


def tans_spread(q):
    """State of the k-th visit is k*1283 mod L; visits go to symbols in
    increasing order, q[s] each."""
    L = 1 << TANS_LOG
    owner = []
    for s, v in enumerate(q):
        owner.extend([s] * v)
    spread = [0] * L
    for k in range(L):
        spread[(k * TANS_STEP) % L] = owner[k]
    return spread


def tans_encode_segment(q, syms):
    """Returns (list of bits, decoding order, the 11 state bits first)."""
    L = 1 << TANS_LOG
    spread = tans_spread(q)
    states = {}
    for x in range(L):
        states.setdefault(spread[x], []).append(x)
    X = L
    chunks = []
    for s in reversed(syms):
        nb = 0
        while (X >> nb) >= 2 * q[s]:
            nb += 1
        chunks.append([(X >> i) & 1 for i in range(nb)])
        X = L + states[s][(X >> nb) - q[s]]
    bits = [((X - L) >> i) & 1 for i in range(TANS_LOG)]
    for c in reversed(chunks):
        bits.extend(c)
    return bits


def tans_decode_segment(q, bits, n):
    L = 1 << TANS_LOG
    spread = tans_spread(q)
    rank, seen = [0] * L, {}
    for x in range(L):
        rank[x] = seen.get(spread[x], 0)
        seen[spread[x]] = rank[x] + 1
    pos = TANS_LOG
    X = L + sum(b << i for i, b in enumerate(bits[:TANS_LOG]))
    out = []
    for _ in range(n):
        x = X - L
        s = spread[x]
        y = q[s] + rank[x]
        nb = TANS_LOG - (y.bit_length() - 1)
        v = sum(b << i for i, b in enumerate(bits[pos:pos + nb]))
        if len(bits[pos:pos + nb]) < nb:
            raise ValueError("segment too short")
        pos += nb
        out.append(s)
        X = (y << nb) + v
    if X != L or pos != len(bits):
        raise ValueError("segment does not end in the initial state")
    return out


def encode_stream_tans(syms, k, S):
    """One stream section with the tANS coder (no group tables)."""
    n = len(syms)
    A = 1 << k
    h = [0] * A
    for s in syms:
        h[s] += 1
    nseg = (n + S - 1) // S
    present = [s for s in range(A) if h[s]]
    if len(present) == 1:
        return encode_stream(syms, k, S)   # constant
    q = tans_normalize(h)
    segbits = [tans_encode_segment(q, [syms[i] for i in segment_order(n, nseg, j)]) for j in range(nseg)]
    bits = sum(len(b) for b in segbits)
    rh, rp = section(RAW, k, n, nseg, 0)
    th, tp = section(TANS, k, n, nseg, bits, len(present))
    if th + a16(tp) >= rh + a16(rp):
        return encode_stream(syms, k, S, force_raw=True)
    out = bytearray(th + a16(tp))
    struct.pack_into("<BBHI", out, 0, TANS, 0, nseg, tp)
    pos = 8
    for s in present:
        out[pos + s // 8] |= 1 << (s % 8)
    pos += A // 8
    for s in present:
        struct.pack_into("<H", out, pos, q[s])
        pos += 2
    bw = Bits()
    for j, b in enumerate(segbits):
        struct.pack_into("<H", out, pos + 2 * j, len(b))
        for bit in b:
            bw.put(bit)
    if tp:
        out[th:th + tp] = bw.tobytes(tp)
    return bytes(out)


# ------------------------------------------------- packed exponent pairs ----
# Restated from the codec's reading of NeuralZip's packed exponents: in each
# 32-value strip, values 2i and 2i+1 are a pair position; a group's pair code
# has F (its 16 most common values, most common first, ties to the smaller
# value), tokens 0..255 for single values and 256 + 16*rank(x) + rank(y) for
# a pair of values of F, and one length per token.
def pair_F(pooled):
    order = sorted((s for s in range(256) if pooled[s]), key=lambda s: (-pooled[s], s))
    return order[:16]


def strip_tokens(vals, F, tlen):
    rank = {v: i for i, v in enumerate(F)}
    toks, i = [], 0
    while i < len(vals):
        if i + 1 < len(vals):
            x, y = vals[i], vals[i + 1]
            if x in rank and y in rank and tlen[256 + 16 * rank[x] + rank[y]]:
                toks.append(256 + 16 * rank[x] + rank[y])
            else:
                toks += [x, y]
            i += 2
        else:
            toks.append(vals[i])
            i += 1
    return toks


def pair_setup(chunks, gmap, K, single_lens):
    """chunks: the exponent list of every chunk; gmap: group of each chunk;
    single_lens: each group's single-value lengths.  Returns per group
    (packs, F, token lengths)."""
    out = []
    for g in range(K):
        pooled = [0] * 256
        for c, ex in enumerate(chunks):
            if gmap[c] == g:
                for v in ex:
                    pooled[v] += 1
        F = pair_F(pooled)
        rank = {v: i for i, v in enumerate(F)}
        counts = [0] * 512
        for c, ex in enumerate(chunks):
            if gmap[c] != g:
                continue
            for a in range(0, len(ex), 32):
                st = ex[a:a + 32]
                for i in range(0, len(st), 2):
                    if i + 1 < len(st) and st[i] in rank and st[i + 1] in rank:
                        counts[256 + 16 * rank[st[i]] + rank[st[i + 1]]] += 1
                    else:
                        for v in st[i:i + 2]:
                            counts[v] += 1
        tlen = group_lengths(counts)
        tok_bits = sum(c * l for c, l in zip(counts, tlen))
        single_bits = sum(pooled[s] * single_lens[g][s] for s in range(256))
        out.append((tok_bits < single_bits, F, tlen))
    return out


def encode_stream(syms, k, S, group=None, force_raw=False):
    """One stream section; group = (lengths, id) or (lengths, id, (F, token
    lengths)) to try GROUP mode (with pair tokens)."""
    n = len(syms)
    A = 1 << k
    h = [0] * A
    for s in syms:
        h[s] += 1
    nseg = (n + S - 1) // S
    present = [s for s in range(A) if h[s]]
    if len(present) == 1:
        mode, aux, lens = CONST, present[0], None
    else:
        rh, rp = section(RAW, k, n, nseg, 0)
        raw_size = rh + a16(rp)
        mode, aux, lens = RAW, 0, None
        tried = False
        if group is not None and len(group) == 3:
            gl, gid, (F, tlen) = group
            toks = [t for a in range(0, n, 32) for t in strip_tokens(syms[a:a + 32], F, tlen)]
            if all(tlen[t] > 0 for t in toks):
                tried = True
                bits = sum(tlen[t] for t in toks)
                gh, gp = section(GROUP, k, n, nseg, bits)
                if gh + a16(gp) >= raw_size:
                    return encode_stream(syms, k, S, None, force_raw=True)
                out = bytearray(gh + a16(gp))
                struct.pack_into("<BBHI", out, 0, GROUP, gid, nseg, gp)
                codes = canonical(tlen)
                bw = Bits()
                for j in range(nseg):
                    b0 = bw.n
                    for a in range(j * 32, n, nseg * 32):
                        for t in strip_tokens(syms[a:a + 32], F, tlen):
                            bw.code(codes[t], tlen[t])
                    struct.pack_into("<H", out, 8 + 2 * j, bw.n - b0)
                if gp:
                    out[gh:gh + gp] = bw.tobytes(gp)
                return bytes(out)
        elif group is not None:
            gl, gid = group
            if all(gl[s] > 0 for s in present):
                tried = True
                bits = sum(h[s] * gl[s] for s in range(A))
                gh, gp = section(GROUP, k, n, nseg, bits)
                if gh + a16(gp) < raw_size:
                    mode, aux, lens = GROUP, gid, list(gl)
        if not tried and not force_raw:
            ln = package_merge(h)
            bits = sum(h[s] * ln[s] for s in range(A))
            hh, hp = section(HUFF, k, n, nseg, bits)
            if hh + a16(hp) < raw_size:
                mode, lens = HUFF, ln
    bits = sum(h[s] * lens[s] for s in range(A)) if lens else 0
    head, pay = section(mode, k, n, nseg, bits)
    out = bytearray(head + a16(pay))
    struct.pack_into("<BBHI", out, 0, mode, aux, nseg, pay)
    pos = 8
    if mode == HUFF:
        for s in range(0, A, 2):
            out[pos + s // 2] = lens[s] | (lens[s + 1] << 4)
        pos += A // 2
    bw = Bits()
    if mode in (HUFF, GROUP):
        codes = canonical(lens)
        for j in range(nseg):
            b0 = bw.n
            for i in segment_order(n, nseg, j):
                bw.code(codes[syms[i]], lens[syms[i]])
            struct.pack_into("<H", out, pos + 2 * j, bw.n - b0)
    elif mode == RAW:
        for s in syms:
            bw.value(s, k)
    if pay:
        out[head:head + pay] = bw.tobytes(pay)
    return bytes(out)


def encode_container(dt, tensors, chunk_bytes, groups=None, ts_hash=0, tans=False):
    """tensors: lists of ints (bit patterns); groups: (lengths per group, map)
    or (lengths per group, map, pair codes per group as pair_setup gives);
    tans: the exponent stream with the tANS coder."""
    T = len(tensors)
    ce = chunk_bytes // ESIZE[dt]
    nch = [(len(t) + ce - 1) // ce for t in tensors]
    M = sum(nch)
    off_dir = 64 + 16 * T
    cur = a16(off_dir + 8 * (M + 1))
    raw_off = []
    raw_size = {0: lambda n: n, 1: lambda n: 0, 2: lambda n: (n + 7) // 8, 3: lambda n: (n + 3) // 4}[dt]
    for t in tensors:
        raw_off.append(cur)
        cur = a16(cur + raw_size(len(t)))
    off_rec = cur
    recs, c = [], 0
    for ti, t in enumerate(tensors):
        for i0 in range(0, len(t), ce):
            chunk = t[i0:i0 + ce]
            planes = [[] for _ in range(NCODED[dt])]
            for w in chunk:
                sy, _ = split(dt, w)
                for p in range(NCODED[dt]):
                    planes[p].append(sy[p])
            rec = b""
            for p in range(NCODED[dt]):
                grp = None
                if groups is not None and p == 0:
                    g = groups[1][c]
                    grp = (groups[0][g], g)
                    if len(groups) == 3 and groups[2][g][0]:
                        grp = (groups[0][g], g, (groups[2][g][1], groups[2][g][2]))
                if tans and p == 0:
                    rec += encode_stream_tans(planes[p], kbits(dt, p), SEG[dt])
                else:
                    rec += encode_stream(planes[p], kbits(dt, p), SEG[dt], grp)
            recs.append(rec)
            c += 1
    total = off_rec + sum(len(r) for r in recs) + 16
    out = bytearray(total)
    struct.pack_into("<IHBBIIQIHBBQQQQ", out, 0, 0x31464E5A, 1, dt, 1 if groups else 0, T,
                     chunk_bytes, sum(len(t) for t in tensors), M, SEG[dt], MAX_LEN, NCODED[dt],
                     ts_hash if groups else 0, off_dir, off_rec, total)
    for ti, t in enumerate(tensors):
        struct.pack_into("<QQ", out, 64 + 16 * ti, len(t), raw_off[ti])
        for i, w in enumerate(t):
            _, raw = split(dt, w)
            if dt == 0:
                out[raw_off[ti] + i] = raw
            elif dt == 2 and raw:
                out[raw_off[ti] + i // 8] |= 1 << (i % 8)
            elif dt == 3 and raw:
                out[raw_off[ti] + i // 4] |= raw << (2 * (i % 4))
    pos = off_rec
    for ci, r in enumerate(recs):
        struct.pack_into("<Q", out, off_dir + 8 * ci, pos)
        out[pos:pos + len(r)] = r
        pos += len(r)
    struct.pack_into("<Q", out, off_dir + 8 * M, pos)
    return bytes(out)


def decode_container(blob, group_lengths_table=None, pair_codes=None):
    """Parses and decodes a container; returns the list of tensors (ints).
    pair_codes: per group (packs, F, token lengths), as pair_setup gives."""
    (magic, ver, dt, flags, T, cb, ntot, M, S, L, nc, h, off_dir, off_rec,
     total) = struct.unpack_from("<IHBBIIQIHBBQQQQ", blob, 0)
    assert magic == 0x31464E5A and ver == 1 and L == MAX_LEN
    ce = cb // ESIZE[dt]
    outs, c = [], 0
    for ti in range(T):
        n, roff = struct.unpack_from("<QQ", blob, 64 + 16 * ti)
        vals = []
        for i0 in range(0, n, ce):
            m = min(ce, n - i0)
            pos = struct.unpack_from("<Q", blob, off_dir + 8 * c)[0]
            planes = []
            for p in range(nc):
                k = kbits(dt, p)
                A = 1 << k
                mode, aux, nseg, pay = struct.unpack_from("<BBHI", blob, pos)
                q = pos + 8
                syms = []
                if mode == CONST:
                    syms = [aux] * m
                    head = 16
                elif mode == RAW:
                    head = 16
                    v = int.from_bytes(blob[pos + head:pos + head + pay], "little")
                    syms = [(v >> (i * k)) & (A - 1) for i in range(m)]
                elif mode == TANS:
                    assert p == 0
                    present = [s for s in range(A) if (blob[q + s // 8] >> (s % 8)) & 1]
                    q += A // 8
                    cnt = [0] * A
                    for s in present:
                        cnt[s] = struct.unpack_from("<H", blob, q)[0]
                        q += 2
                    seg_bits = [struct.unpack_from("<H", blob, q + 2 * j)[0] for j in range(nseg)]
                    head = a16(q + 2 * nseg - pos)
                    v = int.from_bytes(blob[pos + head:pos + head + pay], "little")
                    bitpos = 0
                    syms = [None] * m
                    for j in range(nseg):
                        seg = [(v >> (bitpos + i)) & 1 for i in range(seg_bits[j])]
                        bitpos += seg_bits[j]
                        order = list(segment_order(m, nseg, j))
                        for i, sy in zip(order, tans_decode_segment(cnt, seg, len(order))):
                            syms[i] = sy
                else:
                    if mode == HUFF:
                        lens = []
                        for s in range(0, A, 2):
                            lens += [blob[q + s // 2] & 15, blob[q + s // 2] >> 4]
                        q += A // 2
                    else:
                        lens = list(group_lengths_table[aux])
                        if pair_codes is not None and pair_codes[aux][0]:
                            _, F, tlen = pair_codes[aux]
                            seg_bits = [struct.unpack_from("<H", blob, q + 2 * j)[0] for j in range(nseg)]
                            head = a16(q + 2 * nseg - pos)
                            codes = canonical(tlen)
                            table = {(tlen[t], codes[t]): t for t in range(512) if tlen[t]}
                            v = int.from_bytes(blob[pos + head:pos + head + pay], "little")
                            bitpos, syms = 0, [None] * m
                            for j in range(nseg):
                                end = bitpos + seg_bits[j]
                                order = list(segment_order(m, nseg, j))
                                got = []
                                while len(got) < len(order):
                                    code, l = 0, 0
                                    while True:
                                        code = (code << 1) | ((v >> bitpos) & 1)
                                        bitpos += 1
                                        l += 1
                                        if (l, code) in table:
                                            t = table[(l, code)]
                                            break
                                        assert l < MAX_LEN
                                    got += [t] if t < 256 else [F[(t - 256) >> 4], F[(t - 256) & 15]]
                                assert len(got) == len(order) and bitpos == end
                                for i, val in zip(order, got):
                                    syms[i] = val
                            planes.append(syms)
                            pos += head + a16(pay)
                            continue
                    seg_bits = [struct.unpack_from("<H", blob, q + 2 * j)[0] for j in range(nseg)]
                    head = a16(q + 2 * nseg - pos)
                    codes = canonical(lens)
                    table = {(lens[s], codes[s]): s for s in range(A) if lens[s]}
                    v = int.from_bytes(blob[pos + head:pos + head + pay], "little")
                    bitpos = 0
                    syms = [None] * m
                    for j in range(nseg):
                        end = bitpos + seg_bits[j]
                        for i in segment_order(m, nseg, j):
                            code, l = 0, 0
                            while True:
                                code = (code << 1) | ((v >> bitpos) & 1)
                                bitpos += 1
                                l += 1
                                if (l, code) in table:
                                    syms[i] = table[(l, code)]
                                    break
                                assert l < MAX_LEN
                        assert bitpos == end
                planes.append(syms)
                pos += head + a16(pay)
            for i in range(m):
                e = i0 + i
                if dt == 0:
                    raw = blob[roff + e]
                elif dt == 2:
                    raw = (blob[roff + e // 8] >> (e % 8)) & 1
                elif dt == 3:
                    raw = (blob[roff + e // 4] >> (2 * (e % 4))) & 3
                else:
                    raw = 0
                vals.append(merge(dt, [planes[p][i] for p in range(nc)], raw))
            c += 1
        outs.append(vals)
    return outs
