/*
 * zno.c -- CPU oracle of the exponent-Huffman float codec.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  Plain, scalar,
 * single-threaded C; every step is written in the order the method states it,
 * with no blocking, fusion or reordering.  Bits are written and read one at a
 * time.  Speed is not a goal.
 *
 * Sources (page titles and sections; no text is quoted):
 *  [T599]  THEORY-599, nucleation note on "ZipNN: Lossless Compression for AI
 *          Models": "What was actually shown" -- exponent distribution (ZipNN
 *          Fig. 2), per-field compressibility (ZipNN Table II), order-0 only
 *          (ZipNN section III-A b), implied entropy.
 *  [FP8]   "Lossless Compression of Neural Network Components: Weights,
 *          Checkpoints, and K/V Caches in Low-Precision Formats", Abstract.
 *  [NZ]    "NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract.
 *  [ZNN]   "ZipNN: Lossless Compression for AI Models", Abstract (arXiv).
 * Textbook methods named where used: package-merge (Larmore and Hirschberg,
 * 1990) for optimal length-limited prefix codes; canonical codes and LSB-first
 * bit packing as specified in RFC 1951 sections 3.1.1 and 3.2.2.
 *
 * ---------------------------------------------------------------------------
 * FORMAT (version 1).  Readings of what the pages leave open are marked R#.
 *
 * R1 Field split (what "extract the exponent" means) [T599 Table II; FP8]:
 *    BF16 word w:  E  = (w>>7)&0xFF                      coded stream 0
 *                  SF = ((w>>8)&0x80) | (w&0x7F)         always-raw byte plane
 *    FP32 word w:  P0 = (w>>23)&0xFF                     coded stream 0
 *                  P1 = ((w>>24)&0x80) | ((w>>16)&0x7F)  coded stream 1
 *                  P2 = (w>>8)&0xFF, P3 = w&0xFF         coded streams 2, 3
 *    FP8 byte b:   E4 = (b>>3)&0xF (stream 0), M3 = b&7 (stream 1),
 *                  S = b>>7 (always-raw bit plane).
 *    FP4 (E2M1, the FP8 page's other low-precision format), stored two
 *    values to a byte, the first in the low nibble; a nibble is
 *    sign(bit 3) | exponent(bits 2..1) | mantissa(bit 0).  One element is
 *    one byte (two values): E = e_lo | e_hi<<2 (stream 0, 4 bits),
 *    M = m_lo | m_hi<<1 (stream 1, 2 bits), S = s_lo | s_hi<<1 (always-raw,
 *    2 bits per element).  Reading: the pages name FP4 but not its layout;
 *    this is its usual packed storage, with each field of the byte's two
 *    values kept together as one symbol.
 *    Every bit pattern is data: NaN, Inf, subnormals and -0 are not special.
 * R2 Chunks: a chunk holds chunk_bytes of uncompressed input of ONE tensor;
 *    the last chunk of a tensor may be short.  A coded stream of n symbols
 *    has nseg = ceil(n / S) segments (S = 512 for BF16, 256 for FP32, 1024
 *    for FP8: a full 256 KiB chunk gives 256 segments per coded stream).  The stream is cut into strips of W = 32 consecutive symbols
 *    (the last strip may be short); segment j holds strips j, j + nseg,
 *    j + 2*nseg, ... in that order.  A full chunk gives every segment S/W
 *    strips.
 * R3 Code: optimal prefix code with lengths <= L = 11 (package-merge),
 *    leaves ordered by (count, symbol), leaves before packages at equal
 *    weight, packages in creation order.  Canonical code assignment.
 * R4 Bits: LSB-first -- stream bit i is bit (i mod 8) of byte i/8.  A Huffman
 *    code word is emitted first-code-bit first; a raw k-bit value is emitted
 *    value-bit-0 first (so raw 8-bit planes are plain bytes).  The segments of
 *    one stream follow each other with no padding between them.
 * R5 Mode per (chunk, coded stream): one distinct symbol -> CONST; else the
 *    smaller of HUFF and RAW by exact section size (ties go to RAW).  With a
 *    group tableset, stream 0 uses GROUP (vs RAW) when the group's table
 *    covers every symbol present, otherwise the chunk is an escape and takes
 *    the HUFF-vs-RAW rule.
 * R6 Container, all integers little-endian:
 *    header (64 B): u32 magic "ZNF1", u16 version=1, u8 dtype, u8 flags
 *      (bit0: group tableset in use), u32 n_tensors, u32 chunk_bytes,
 *      u64 n_elems (all tensors), u32 n_chunks, u16 S, u8 L, u8 n_coded,
 *      u64 tableset hash (0 when bit0 is clear), u64 off_dir,
 *      u64 off_records, u64 total_bytes.
 *    tensor table at 64: per tensor {u64 n_elems, u64 raw_off}.
 *    directory at off_dir: u64 record offset [n_chunks + 1].
 *    always-raw sections (BF16 SF bytes, FP8 sign bits), one per tensor,
 *      each 16-byte aligned.
 *    records from off_records, chunk order = tensor order, then 16 zero bytes.
 *    A record is, per coded stream in order, a section:
 *      u8 mode, u8 aux (CONST symbol / group id), u16 n_seg, u32 payload_bytes;
 *      [HUFF] code lengths, two per byte (even symbol in the low nibble);
 *      [HUFF, GROUP] u16 bit length of each segment;
 *      zero pad to 16 B; payload; zero pad to 16 B.
 *    payload_bytes: HUFF/GROUP 4*ceil(bits/32); RAW ceil(n*k/8); CONST 0.
 * R7 Setup (NeuralZip grouping), all integer: key = floor(sum(s*h[s])*2^16/n)
 *    orders the chunks; K contiguous groups cut at floor(M*g/K); then 8
 *    rounds of (tables from pooled histograms, reassign each chunk to the
 *    table of least coded size, ties to the smaller group id); final tables
 *    from the final assignment.  A pooled histogram with one symbol gets the
 *    smallest absent symbol as a zero-weight second leaf.  The chunk->group
 *    map is positional (tensor order, chunk order).
 * R8 tANS coder of the exponent stream (the alternative entropy stage of
 *    THEORY-599's order-0 discussion, ZipNN Fig. 4: FSE, a tabled
 *    asymmetric-numeral-system coder, codes exponents 0-2% smaller than
 *    Huffman).  Chosen per compression call, for chunks coded with their own
 *    table (no group tables).  Ours, after Duda's tabled ANS:
 *    - 2^11 states.  Normalised counts q: q[s] = max(1, floor(h[s]*2^11/n))
 *      for present symbols (0 otherwise); if they sum below 2^11 the
 *      shortfall goes one each to the present symbols of largest remainder
 *      h[s]*2^11 mod n (ties to the smaller symbol); if above, one is taken
 *      repeatedly from the symbol of largest q (ties to the smaller symbol).
 *    - Spread: symbols in increasing order, q[s] states each, visit states
 *      0, 1283, 2*1283, ... modulo 2^11 (1283 is odd, so every state once).
 *    - A symbol s seen at state x in [0, 2^11) has rank r = number of states
 *      below x that hold s; decoding at X = 2^11 + x outputs s, forms
 *      y = q[s] + r, reads nb = 11 - floor(log2 y) bits v (value bit 0 first)
 *      and moves to X = y*2^nb + v.  Encoding runs the segment backwards from
 *      X = 2^11: for s it emits the nb low bits of X with X >> nb in
 *      [q[s], 2q[s]) and moves to 2^11 + (the (X>>nb) - q[s])-th state of s.
 *      A segment's bits are its final state minus 2^11 (11 bits), then the
 *      emitted bits in decoding order (the first symbol's first), so it
 *      decodes forward from that state and must end at 2^11 having read
 *      exactly its bit length.
 *    - Mode TANS (4) when its section is smaller than the raw one (ties to
 *      RAW); one distinct symbol is CONST as always.  Section: head, a
 *      presence mask of A bits (bit s of byte s/8), u16 q[s] of each present
 *      symbol in increasing order, u16 bit length per segment, pad 16,
 *      payload (4*ceil(bits/32) bytes, segments bit-contiguous), pad 16.
 * R9 Packed exponent pairs ("NeuralZip", Abstract: recurring exponent tuples
 *    represented by packed exponents, chosen by the setup, for a further
 *    moderate gain).  Ours, for BF16 setups with groups when asked for:
 *    - pair positions: in each 32-value strip of a chunk's exponent stream,
 *      values 2i and 2i+1 (a strip of odd length ends with a lone value);
 *    - after the grouping, per group: F = the (up to) 16 values of largest
 *      pooled count (ties to the smaller value; present values only), rank
 *      = position in F; over the group's chunks, a pair position (x, y)
 *      with x, y in F counts for token 256 + 16*rank(x) + rank(y), every
 *      other value for its single token x; token lengths by the R7 rule
 *      over the 512 token counts; the group packs iff the tokens' pooled
 *      bits are fewer than the singles' under its single table (strict);
 *    - a chunk of a packing group coded with its group code: per pair
 *      position the pair token when x, y in F and the token has a code
 *      word, else the two singles; lone values singles; a single without a
 *      code word makes the chunk an escape (own table, no pairs).  Canonical
 *      codes over the 512 tokens, first bit first as always;
 *    - decoding reads tokens in segment order, a pair token giving its two
 *      values; the segment's tokens must give exactly its value count;
 *    - the tableset (format version 2) stores per group the packing flag,
 *      F and the token lengths; a transfer keeps the source's.
 * ---------------------------------------------------------------------------
 */
#include "zno.h"

#include <stdlib.h>
#include <string.h>

#define MAXLEN 11
#define MAGIC 0x31464E5Au
#define TS_MAGIC 0x53544E5Au
#define VERSION 1
#define ROUNDS 8
#define STRIP 32

/* ------------------------------------------------------------------ */
/* geometry of each dtype                                              */
/* ------------------------------------------------------------------ */
static int esize(int dt) { return dt == ZNO_BF16 ? 2 : dt == ZNO_FP32 ? 4 : 1; }
static int ncoded(int dt) { return dt == ZNO_BF16 ? 1 : dt == ZNO_FP32 ? 4 : 2; }
static int kbits(int dt, int p) {
  return dt == ZNO_FP8_E4M3 ? (p == 0 ? 4 : 3) : dt == ZNO_FP4X2_E2M1 ? (p == 0 ? 4 : 2) : 8;
}
static int segsyms(int dt) { return dt == ZNO_BF16 ? 512 : dt == ZNO_FP32 ? 256 : 1024; }
static uint64_t rawplane_bytes(int dt, uint64_t n) {
  return dt == ZNO_BF16 ? n : dt == ZNO_FP8_E4M3 ? (n + 7) / 8 : dt == ZNO_FP4X2_E2M1 ? (n + 3) / 4 : 0;
}
static uint64_t align16(uint64_t x) { return (x + 15) & ~(uint64_t)15; }
static int valid_dtype(int dt) {
  return dt == ZNO_BF16 || dt == ZNO_FP32 || dt == ZNO_FP8_E4M3 || dt == ZNO_FP4X2_E2M1;
}
static int valid_chunk(uint32_t cb) { return cb >= 4096 && cb <= (1u << 20) && cb % 4096 == 0; }

static void put_u16(uint8_t *p, uint32_t v) { p[0] = v & 0xFF; p[1] = (v >> 8) & 0xFF; }
static void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (v >> (8 * i)) & 0xFF; }
static void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (v >> (8 * i)) & 0xFF; }
static uint32_t get_u16(const uint8_t *p) { return p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get_u32(const uint8_t *p) {
  return p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint64_t get_u64(const uint8_t *p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; i--) v = (v << 8) | p[i];
  return v;
}

/* ------------------------------------------------------------------ */
/* R1: field split and merge  [T599 Table II; FP8 Abstract]            */
/* ------------------------------------------------------------------ */
static uint32_t load_elem(int dt, const uint8_t *base, uint64_t i) {
  const uint8_t *p = base + i * (uint64_t)esize(dt);
  if (dt == ZNO_BF16) return p[0] | ((uint32_t)p[1] << 8);
  if (dt == ZNO_FP32) return get_u32(p);
  return p[0];
}
static void store_elem(int dt, uint8_t *base, uint64_t i, uint32_t w) {
  uint8_t *p = base + i * (uint64_t)esize(dt);
  if (dt == ZNO_BF16) { put_u16(p, w); return; }
  if (dt == ZNO_FP32) { put_u32(p, w); return; }
  p[0] = (uint8_t)w;
}

/* Splits one element into its coded symbols and its always-raw bits. */
static void split_one(int dt, uint32_t w, uint8_t *sym, uint32_t *raw) {
  if (dt == ZNO_BF16) {
    sym[0] = (w >> 7) & 0xFF;                       /* biased exponent, 8 bits   */
    *raw = ((w >> 8) & 0x80) | (w & 0x7F);          /* sign | 7 fraction bits    */
  } else if (dt == ZNO_FP32) {
    sym[0] = (w >> 23) & 0xFF;                      /* biased exponent           */
    sym[1] = ((w >> 24) & 0x80) | ((w >> 16) & 0x7F); /* sign | fraction[22:16] */
    sym[2] = (w >> 8) & 0xFF;                       /* fraction[15:8]            */
    sym[3] = w & 0xFF;                              /* fraction[7:0]             */
    *raw = 0;
  } else if (dt == ZNO_FP8_E4M3) {
    sym[0] = (w >> 3) & 0xF;                        /* E4M3 exponent             */
    sym[1] = w & 7;                                 /* E4M3 mantissa             */
    *raw = (w >> 7) & 1;                            /* sign                      */
  } else {                                          /* two E2M1 values, low first */
    const uint32_t lo = w & 0xF, hi = (w >> 4) & 0xF;
    sym[0] = (uint8_t)(((lo >> 1) & 3) | (((hi >> 1) & 3) << 2));  /* exponents   */
    sym[1] = (uint8_t)((lo & 1) | ((hi & 1) << 1));                /* mantissas   */
    *raw = ((lo >> 3) & 1) | (((hi >> 3) & 1) << 1);               /* signs       */
  }
}
static uint32_t merge_one(int dt, const uint8_t *sym, uint32_t raw) {
  if (dt == ZNO_BF16)
    return ((raw & 0x80) << 8) | ((uint32_t)sym[0] << 7) | (raw & 0x7F);
  if (dt == ZNO_FP32)
    return ((uint32_t)(sym[1] & 0x80) << 24) | ((uint32_t)sym[0] << 23) |
           ((uint32_t)(sym[1] & 0x7F) << 16) | ((uint32_t)sym[2] << 8) | sym[3];
  if (dt == ZNO_FP8_E4M3) return ((raw & 1) << 7) | ((uint32_t)(sym[0] & 0xF) << 3) | (sym[1] & 7);
  const uint32_t lo = ((raw & 1) << 3) | ((uint32_t)(sym[0] & 3) << 1) | (sym[1] & 1);
  const uint32_t hi = (((raw >> 1) & 1) << 3) | ((uint32_t)((sym[0] >> 2) & 3) << 1) | ((sym[1] >> 1) & 1);
  return lo | (hi << 4);
}

void zno_split(int dt, const void *in, uint64_t n, uint8_t *planes, uint8_t *rawbits) {
  const uint8_t *b = (const uint8_t *)in;
  for (uint64_t i = 0; i < n; i++) {
    uint8_t sym[4];
    uint32_t raw;
    split_one(dt, load_elem(dt, b, i), sym, &raw);
    for (int p = 0; p < ncoded(dt); p++) planes[(uint64_t)p * n + i] = sym[p];
    if (rawbits) rawbits[i] = (uint8_t)raw;
  }
}
void zno_merge(int dt, const uint8_t *planes, const uint8_t *rawbits, uint64_t n, void *out) {
  for (uint64_t i = 0; i < n; i++) {
    uint8_t sym[4] = {0, 0, 0, 0};
    for (int p = 0; p < ncoded(dt); p++) sym[p] = planes[(uint64_t)p * n + i];
    store_elem(dt, (uint8_t *)out, i, merge_one(dt, sym, rawbits ? rawbits[i] : 0));
  }
}

/* ------------------------------------------------------------------ */
/* R3: optimal length-limited code lengths by package-merge            */
/* (Larmore and Hirschberg 1990, the "coin collector" formulation).    */
/* Order-0 Huffman coding of the exponent is the method's coder        */
/* [T599, order-0 only; FP8 Abstract]; the length limit is ours.       */
/* ------------------------------------------------------------------ */
typedef struct {
  uint64_t w;
  int sym;    /* >= 0: a leaf (coin of that symbol); -1: a package */
  int c0, c1; /* package: the two items of the previous list it joins */
} pm_item;

/* Adds one to the length of every leaf inside item idx of list j. */
static void pm_expand(pm_item **lists, int j, int idx, uint8_t *len) {
  const pm_item *it = &lists[j][idx];
  if (it->sym >= 0) {
    len[it->sym]++;
    return;
  }
  pm_expand(lists, j - 1, it->c0, len);
  pm_expand(lists, j - 1, it->c1, len);
}

/* Leaves (w[i], sym[i]) must already be sorted by (weight, symbol); d >= 2.
 * List 0 holds the coins of the smallest denomination 2^-L (the leaves);
 * list j merges the leaves with the packages formed from adjacent pairs of
 * list j-1; the first 2d-2 items of list L-1 (denomination 1/2) are
 * selected, and each symbol's length is the number of its coins among them. */
static int pm_lengths(const uint64_t *w, const int *sym, int d, int L, uint8_t *len) {
  if (d < 2 || L < 1 || L > 16 || (d > (1 << L))) return ZNO_ERR_ARG;
  pm_item *lists[16];
  int n[16];
  for (int j = 0; j < L; j++) {
    lists[j] = (pm_item *)malloc(sizeof(pm_item) * (size_t)(2 * d));
    if (!lists[j]) {
      for (int q = 0; q < j; q++) free(lists[q]);
      return ZNO_ERR_NOMEM;
    }
  }
  for (int i = 0; i < d; i++) {
    lists[0][i].w = w[i];
    lists[0][i].sym = sym[i];
    lists[0][i].c0 = lists[0][i].c1 = -1;
  }
  n[0] = d;
  for (int j = 1; j < L; j++) {
    int np = n[j - 1] / 2, a = 0, k = 0, o = 0;
    while (a < d || k < np) {
      uint64_t pw = 0;
      if (k < np) pw = lists[j - 1][2 * k].w + lists[j - 1][2 * k + 1].w;
      if (a < d && (k >= np || w[a] <= pw)) { /* leaf first at equal weight */
        lists[j][o].w = w[a];
        lists[j][o].sym = sym[a];
        lists[j][o].c0 = lists[j][o].c1 = -1;
        a++;
      } else {
        lists[j][o].w = pw;
        lists[j][o].sym = -1;
        lists[j][o].c0 = 2 * k;
        lists[j][o].c1 = 2 * k + 1;
        k++;
      }
      o++;
    }
    n[j] = o;
  }
  for (int i = 0; i < d; i++) len[sym[i]] = 0;
  if (n[L - 1] < 2 * d - 2) {
    for (int j = 0; j < L; j++) free(lists[j]);
    return ZNO_ERR_ARG;
  }
  for (int idx = 0; idx < 2 * d - 2; idx++) pm_expand(lists, L - 1, idx, len);
  for (int j = 0; j < L; j++) free(lists[j]);
  return ZNO_OK;
}

/* Sorts the leaves by (count ascending, symbol ascending); insertion sort. */
static void sort_leaves(uint64_t *w, int *sym, int d) {
  for (int i = 1; i < d; i++) {
    uint64_t kw = w[i];
    int ks = sym[i], j = i - 1;
    while (j >= 0 && (w[j] > kw || (w[j] == kw && sym[j] > ks))) {
      w[j + 1] = w[j];
      sym[j + 1] = sym[j];
      j--;
    }
    w[j + 1] = kw;
    sym[j + 1] = ks;
  }
}

/* Code lengths for a histogram; returns the number of distinct symbols d.
 * d < 2 leaves every length 0 (the stream is constant or empty). */
int zno_code_lengths(const uint64_t *h, int A, int L, uint8_t *len) {
  uint64_t w[512];
  int sym[512], d = 0;
  if (A < 2 || A > 512) return ZNO_ERR_ARG;
  memset(len, 0, (size_t)A);
  for (int s = 0; s < A; s++)
    if (h[s]) {
      w[d] = h[s];
      sym[d] = s;
      d++;
    }
  if (d < 2) return d;
  sort_leaves(w, sym, d);
  int rc = pm_lengths(w, sym, d, L, len);
  return rc < 0 ? rc : d;
}

/* Lengths for a pooled group histogram (R7): as above, but one present
 * symbol gets the smallest absent symbol as a zero-weight partner so the
 * table is a complete code; an empty histogram gives an empty table. */
int zno_group_lengths(const uint64_t *h, int A, int L, uint8_t *len) {
  uint64_t w[512];
  int sym[512], d = 0;
  if (A < 2 || A > 512) return ZNO_ERR_ARG;
  memset(len, 0, (size_t)A);
  for (int s = 0; s < A; s++)
    if (h[s]) {
      w[d] = h[s];
      sym[d] = s;
      d++;
    }
  if (d == 0) return 0;
  if (d == 1) {
    int partner = 0;
    while (partner == sym[0]) partner++;
    w[1] = 0;
    sym[1] = partner;
    d = 2;
  }
  sort_leaves(w, sym, d);
  int rc = pm_lengths(w, sym, d, L, len);
  return rc < 0 ? rc : d;
}

/* Canonical code values from lengths (RFC 1951 section 3.2.2). */
void zno_canonical_codes(const uint8_t *len, int A, int L, uint32_t *code) {
  uint32_t bl_count[17] = {0}, next_code[17] = {0}, c = 0;
  for (int s = 0; s < A; s++)
    if (len[s]) bl_count[len[s]]++;
  for (int bits = 1; bits <= L; bits++) {
    c = (c + bl_count[bits - 1]) << 1;
    next_code[bits] = c;
  }
  for (int s = 0; s < A; s++) code[s] = len[s] ? next_code[len[s]]++ : 0;
}

/* ------------------------------------------------------------------ */
/* R4: LSB-first bit writer and reader, one bit at a time              */
/* ------------------------------------------------------------------ */
typedef struct {
  uint8_t *buf;  /* zero-initialised */
  uint64_t pos;  /* bits written */
} bitw;
static void put_bit(bitw *b, unsigned bit) {
  if (bit) b->buf[b->pos >> 3] |= (uint8_t)(1u << (b->pos & 7));
  b->pos++;
}
static void put_code(bitw *b, uint32_t code, int len) { /* first code bit first */
  for (int i = len - 1; i >= 0; i--) put_bit(b, (code >> i) & 1);
}
static void put_value(bitw *b, uint32_t v, int k) { /* value bit 0 first */
  for (int i = 0; i < k; i++) put_bit(b, (v >> i) & 1);
}

typedef struct {
  const uint8_t *buf;
  uint64_t pos, end; /* bit positions */
} bitr;
static int get_bit(bitr *r, unsigned *bit) {
  if (r->pos >= r->end) return -1;
  *bit = (r->buf[r->pos >> 3] >> (r->pos & 7)) & 1;
  r->pos++;
  return 0;
}

/* ------------------------------------------------------------------ */
/* R8: tabled asymmetric numeral systems                               */
/* ------------------------------------------------------------------ */
#define TL (1u << ZNO_TANS_LOG)
#define TSTEP 1283u

int zno_tans_normalize(const uint64_t *h, int A, uint32_t *q) {
  uint64_t n = 0;
  int d = 0;
  if (A < 1 || A > 256) return ZNO_ERR_ARG;
  for (int s = 0; s < A; s++) {
    n += h[s];
    d += h[s] != 0;
  }
  if (n == 0) return ZNO_ERR_ARG;
  int64_t sum = 0;
  for (int s = 0; s < A; s++) {
    q[s] = 0;
    if (!h[s]) continue;
    uint64_t f = h[s] * TL / n;
    q[s] = f ? (uint32_t)f : 1u;
    sum += q[s];
  }
  /* shortfall: one each to the largest remainders (at most d of them) */
  if (sum < (int64_t)TL) {
    /* the floors lose less than one per present symbol, so the shortfall is
       at most d: one pass over the d largest remainders covers it */
    uint8_t given[256] = {0};
    int64_t need = (int64_t)TL - sum;
    for (int64_t k = 0; k < need; k++) {
      int best = -1;
      uint64_t br = 0;
      for (int s = 0; s < A; s++) {
        if (!h[s] || given[s]) continue;
        uint64_t r = (h[s] * TL) % n;
        if (best < 0 || r > br) {
          best = s;
          br = r;
        }
      }
      if (best < 0) return ZNO_ERR_ARG;
      given[best] = 1;
      q[best]++;
      sum++;
    }
  }
  /* excess (from the symbols raised to 1): one at a time from the largest */
  while (sum > (int64_t)TL) {
    int best = -1;
    for (int s = 0; s < A; s++)
      if (q[s] > 1 && (best < 0 || q[s] > q[best])) best = s;
    if (best < 0) return ZNO_ERR_ARG;
    q[best]--;
    sum--;
  }
  return d;
}

void zno_tans_spread(const uint32_t *q, int A, uint8_t *sym_of_state) {
  uint32_t pos = 0;
  for (int s = 0; s < A; s++)
    for (uint32_t i = 0; i < q[s]; i++) {
      sym_of_state[pos] = (uint8_t)s;
      pos = (pos + TSTEP) & (TL - 1);
    }
}

static int floor_log2(uint32_t y) {
  int b = -1;
  while (y) {
    y >>= 1;
    b++;
  }
  return b;
}

int64_t zno_tans_encode(const uint32_t *q, int A, const uint8_t *sym, uint64_t n, uint8_t *out,
                        uint32_t *final_state) {
  uint8_t spread[TL];
  uint32_t first[257], cnt[256];
  uint32_t *state_of = (uint32_t *)malloc(sizeof(uint32_t) * TL); /* [first[s] + k] = k-th state of s */
  uint32_t *cval = (uint32_t *)malloc(sizeof(uint32_t) * (n ? n : 1));
  uint8_t *cbits = (uint8_t *)malloc(n ? n : 1);
  if (!state_of || !cval || !cbits) {
    free(state_of), free(cval), free(cbits);
    return ZNO_ERR_NOMEM;
  }
  zno_tans_spread(q, A, spread);
  first[0] = 0;
  for (int s = 0; s < A; s++) {
    first[s + 1] = first[s] + q[s];
    cnt[s] = 0;
  }
  for (uint32_t x = 0; x < TL; x++) {
    int s = spread[x];
    state_of[first[s] + cnt[s]++] = x;
  }
  /* backwards over the symbols, from the initial state 2^11 */
  uint32_t X = TL;
  int64_t total = 0;
  for (uint64_t i = n; i-- > 0;) {
    int s = sym[i];
    if (s >= A || q[s] == 0) {
      free(state_of), free(cval), free(cbits);
      return ZNO_ERR_ARG;
    }
    int nb = 0;
    while ((X >> nb) >= 2 * q[s]) nb++;
    cval[i] = X & ((1u << nb) - 1u);
    cbits[i] = (uint8_t)nb;
    total += nb;
    X = TL + state_of[first[s] + ((X >> nb) - q[s])];
  }
  *final_state = X - TL;
  /* the bits in decoding order: the first symbol's first, value bit 0 first */
  if (out) {
    bitw bw = {out, 0};
    for (uint64_t i = 0; i < n; i++) put_value(&bw, cval[i], cbits[i]);
  }
  free(state_of), free(cval), free(cbits);
  return total;
}

/* Decodes n symbols of one segment from the bit reader br (positioned at the
 * segment's first bit, ending at its last); spread and rank describe the
 * states (rank[x]: states below x holding the same symbol). */
static int tans_decode_segment(const uint32_t *q, const uint8_t *spread, const uint32_t *rank, bitr *br,
                               uint32_t final_state, uint64_t n, uint8_t *sym, uint64_t stride_fn_unused) {
  (void)stride_fn_unused;
  uint32_t X = TL + final_state;
  for (uint64_t i = 0; i < n; i++) {
    uint32_t x = X - TL;
    int s = spread[x];
    uint32_t y = q[s] + rank[x];
    int nb = ZNO_TANS_LOG - floor_log2(y);
    uint32_t v = 0;
    for (int k = 0; k < nb; k++) {
      unsigned bit;
      if (get_bit(br, &bit)) return ZNO_ERR_CORRUPT;
      v |= (uint32_t)bit << k;
    }
    sym[i] = (uint8_t)s;
    X = (y << nb) + v;
  }
  /* a valid segment ends where it began, having read exactly its bits */
  if (X != TL || br->pos != br->end) return ZNO_ERR_CORRUPT;
  return ZNO_OK;
}

/* The states' ranks of a spread table. */
static void tans_ranks(const uint8_t *spread, uint32_t *rank) {
  uint32_t seen[256] = {0};
  for (uint32_t x = 0; x < TL; x++) rank[x] = seen[spread[x]]++;
}

int zno_tans_decode(const uint32_t *q, int A, const uint8_t *bits, uint64_t nbits,
                    uint32_t final_state, uint64_t n, uint8_t *sym) {
  uint8_t spread[TL];
  uint32_t rank[TL];
  uint64_t sum = 0;
  for (int s = 0; s < A; s++) sum += q[s];
  if (sum != TL || final_state >= TL) return ZNO_ERR_CORRUPT;
  zno_tans_spread(q, A, spread);
  tans_ranks(spread, rank);
  bitr br = {bits, 0, nbits};
  return tans_decode_segment(q, spread, rank, &br, final_state, n, sym, 0);
}

/* ------------------------------------------------------------------ */
/* R5/R6: stream sections and chunk records                           */
/* ------------------------------------------------------------------ */
static uint64_t payload_bytes_of(int mode, int k, uint64_t n, uint64_t bits) {
  if (mode == ZNO_HUFF || mode == ZNO_GROUP || mode == ZNO_TANS) return 4 * ((bits + 31) / 32);
  if (mode == ZNO_RAW) return (n * (uint64_t)k + 7) / 8;
  return 0;
}
/* d: present symbols (used by TANS only) */
static uint64_t head_bytes_d(int mode, int k, int nseg, int d) {
  uint64_t h = 8;
  if (mode == ZNO_HUFF) h += (uint64_t)(1 << k) / 2;
  if (mode == ZNO_HUFF || mode == ZNO_GROUP) h += 2 * (uint64_t)nseg;
  if (mode == ZNO_TANS) h += (uint64_t)(1 << k) / 8 + 2 * (uint64_t)d + 2 * (uint64_t)nseg;
  return align16(h);
}
static uint64_t section_bytes_d(int mode, int k, uint64_t n, int nseg, uint64_t bits, int d) {
  return head_bytes_d(mode, k, nseg, d) + align16(payload_bytes_of(mode, k, n, bits));
}
static uint64_t section_bytes(int mode, int k, uint64_t n, int nseg, uint64_t bits) {
  return section_bytes_d(mode, k, n, nseg, bits, 0);
}
static uint64_t chunk_elems(int dt, uint32_t cb) { return cb / (uint32_t)esize(dt); }
static uint64_t nchunks_of(int dt, uint64_t n, uint32_t cb) {
  uint64_t ce = chunk_elems(dt, cb);
  return (n + ce - 1) / ce;
}

/* The pair code of one group: F's ranks and the token lengths. */
typedef struct {
  int nF;
  uint8_t F[16];
  uint8_t rank[256]; /* rank in F, 0xFF when not in F */
  const uint8_t *tlen;
} pair_code;
/* The tokens of the symbols [a, b) of one strip (R9); returns their number. */
static int strip_tokens(const uint8_t *sym, uint64_t a, uint64_t b, const pair_code *pc, uint16_t *tok) {
  int m = 0;
  for (uint64_t i = a; i < b; i += 2) {
    if (i + 1 < b) {
      int rx = pc->rank[sym[i]], ry = pc->rank[sym[i + 1]];
      if (rx < pc->nF && ry < pc->nF && pc->tlen[256 + 16 * rx + ry]) {
        tok[m++] = (uint16_t)(256 + 16 * rx + ry);
        continue;
      }
      tok[m++] = sym[i];
      tok[m++] = sym[i + 1];
    } else {
      tok[m++] = sym[i];
    }
  }
  return m;
}

/* Plans one coded stream of one chunk: histogram, mode and code lengths. */
typedef struct {
  int mode, aux, nseg, d;
  uint8_t len[256];
  uint32_t q[256];  /* TANS: normalised counts */
  uint64_t bits;
  const pair_code *pc; /* GROUP with a packing group (R9) */
} stream_plan;

/* The symbols of segment j of a stream of n symbols, in decoding order
 * (strips j, j + nseg, ...); returns their number. */
static uint64_t segment_symbols(const uint8_t *sym, uint64_t n, int nseg, int j, uint8_t *dst) {
  uint64_t m = 0;
  for (uint64_t q0 = (uint64_t)j * STRIP; q0 < n; q0 += (uint64_t)nseg * STRIP)
    for (uint64_t i = q0; i < n && i < q0 + STRIP; i++) dst[m++] = sym[i];
  return m;
}

static int plan_stream(const uint8_t *sym, uint64_t n, int k, int S, const uint8_t *group_len,
                       int group_id, int coder, const pair_code *pc, stream_plan *pl, int *escape) {
  uint64_t h[256] = {0};
  int A = 1 << k, d = 0, last = 0;
  for (uint64_t i = 0; i < n; i++) h[sym[i]]++;
  for (int s = 0; s < A; s++)
    if (h[s]) {
      d++;
      last = s;
    }
  memset(pl->len, 0, sizeof pl->len);
  pl->pc = NULL;
  pl->d = d;
  pl->nseg = (int)((n + (uint64_t)S - 1) / (uint64_t)S);
  pl->bits = 0;
  pl->aux = 0;
  if (d == 1) {
    pl->mode = ZNO_CONST;
    pl->aux = last;
    return ZNO_OK;
  }
  uint64_t raw = section_bytes(ZNO_RAW, k, n, pl->nseg, 0);
  if (group_len) {
    int covered = 1;
    uint64_t bits = 0;
    if (pc) {
      /* R9: the strips' tokens under the group's pair code */
      uint16_t tok[STRIP];
      for (uint64_t a = 0; a < n; a += STRIP) {
        int m = strip_tokens(sym, a, a + STRIP < n ? a + STRIP : n, pc, tok);
        for (int i = 0; i < m; i++) {
          if (!pc->tlen[tok[i]]) covered = 0;
          bits += pc->tlen[tok[i]];
        }
      }
    } else {
      for (int s = 0; s < A; s++) {
        if (h[s] && !group_len[s]) covered = 0;
        bits += h[s] * group_len[s];
      }
    }
    if (covered) {
      uint64_t gs = section_bytes(ZNO_GROUP, k, n, pl->nseg, bits);
      if (gs < raw) {
        pl->mode = ZNO_GROUP;
        pl->aux = group_id;
        memcpy(pl->len, group_len, (size_t)A);
        pl->pc = pc;
        pl->bits = bits;
      } else {
        pl->mode = ZNO_RAW;
      }
      return ZNO_OK;
    }
    if (escape) *escape = 1;
  }
  if (coder == ZNO_CODER_TANS) {
    /* tANS: exact size from encoding every segment (R8) */
    int rc = zno_tans_normalize(h, A, pl->q);
    if (rc < 0) return rc;
    uint8_t *seg = (uint8_t *)malloc((size_t)n);
    if (!seg) return ZNO_ERR_NOMEM;
    uint64_t bits = 0;
    for (int j = 0; j < pl->nseg; j++) {
      uint64_t m = segment_symbols(sym, n, pl->nseg, j, seg);
      uint32_t st;
      int64_t b = zno_tans_encode(pl->q, A, seg, m, NULL, &st);
      if (b < 0) {
        free(seg);
        return (int)b;
      }
      bits += ZNO_TANS_LOG + (uint64_t)b;   /* the state, then the emitted bits */
    }
    free(seg);
    if (section_bytes_d(ZNO_TANS, k, n, pl->nseg, bits, d) < raw) {
      pl->mode = ZNO_TANS;
      pl->bits = bits;
    } else {
      pl->mode = ZNO_RAW;
    }
    return ZNO_OK;
  }
  uint8_t len[256];
  int rc = zno_code_lengths(h, A, MAXLEN, len);
  if (rc < 0) return rc;
  uint64_t bits = 0;
  for (int s = 0; s < A; s++) bits += h[s] * len[s];
  uint64_t hs = section_bytes(ZNO_HUFF, k, n, pl->nseg, bits);
  if (hs < raw) {
    pl->mode = ZNO_HUFF;
    memcpy(pl->len, len, (size_t)A);
    pl->bits = bits;
  } else {
    pl->mode = ZNO_RAW;
  }
  return ZNO_OK;
}

/* Writes one stream section at out (zeroed); returns its size. */
static uint64_t write_stream(uint8_t *out, const uint8_t *sym, uint64_t n, int k,
                             const stream_plan *pl) {
  int A = 1 << k;
  uint64_t head = head_bytes_d(pl->mode, k, pl->nseg, pl->d);
  uint64_t pay = payload_bytes_of(pl->mode, k, n, pl->bits);
  out[0] = (uint8_t)pl->mode;
  out[1] = (uint8_t)pl->aux;
  put_u16(out + 2, (uint32_t)pl->nseg);
  put_u32(out + 4, (uint32_t)pay);
  uint8_t *q = out + 8;
  if (pl->mode == ZNO_HUFF) {
    for (int s = 0; s < A; s += 2) q[s / 2] = (uint8_t)(pl->len[s] | (pl->len[s + 1] << 4));
    q += A / 2;
  }
  bitw bw = {out + head, 0};
  if (pl->mode == ZNO_GROUP && pl->pc) {
    /* R9: tokens, canonical codes over the 512 tokens */
    uint32_t code[512];
    uint16_t tok[STRIP];
    zno_canonical_codes(pl->pc->tlen, 512, MAXLEN, code);
    for (int j = 0; j < pl->nseg; j++) {
      uint64_t b0 = bw.pos;
      for (uint64_t q0 = (uint64_t)j * STRIP; q0 < n; q0 += (uint64_t)pl->nseg * STRIP) {
        int m = strip_tokens(sym, q0, q0 + STRIP < n ? q0 + STRIP : n, pl->pc, tok);
        for (int i = 0; i < m; i++) put_code(&bw, code[tok[i]], pl->pc->tlen[tok[i]]);
      }
      put_u16(q + 2 * j, (uint32_t)(bw.pos - b0));
    }
  } else if (pl->mode == ZNO_HUFF || pl->mode == ZNO_GROUP) {
    uint32_t code[256];
    zno_canonical_codes(pl->len, A, MAXLEN, code);
    for (int j = 0; j < pl->nseg; j++) {
      uint64_t b0 = bw.pos;
      for (uint64_t q0 = (uint64_t)j * STRIP; q0 < n; q0 += (uint64_t)pl->nseg * STRIP)
        for (uint64_t i = q0; i < n && i < q0 + STRIP; i++)
          put_code(&bw, code[sym[i]], pl->len[sym[i]]);
      put_u16(q + 2 * j, (uint32_t)(bw.pos - b0));
    }
  } else if (pl->mode == ZNO_TANS) {
    for (int s = 0; s < A; s++)
      if (pl->q[s]) q[s / 8] |= (uint8_t)(1u << (s % 8));
    q += A / 8;
    for (int s = 0; s < A; s++)
      if (pl->q[s]) {
        put_u16(q, pl->q[s]);
        q += 2;
      }
    uint8_t *seg = (uint8_t *)malloc((size_t)n), *tmp = (uint8_t *)calloc((size_t)n * 2 + 8, 1);
    for (int j = 0; j < pl->nseg && seg && tmp; j++) {
      uint64_t m = segment_symbols(sym, n, pl->nseg, j, seg);
      uint32_t st;
      memset(tmp, 0, (size_t)n * 2 + 8);
      int64_t b = zno_tans_encode(pl->q, A, seg, m, tmp, &st);
      put_value(&bw, st, ZNO_TANS_LOG);
      for (int64_t i = 0; i < b; i++) put_bit(&bw, (tmp[i >> 3] >> (i & 7)) & 1);
      put_u16(q + 2 * j, (uint32_t)(ZNO_TANS_LOG + b));
    }
    free(seg);
    free(tmp);
  } else if (pl->mode == ZNO_RAW) {
    for (uint64_t i = 0; i < n; i++) put_value(&bw, sym[i], k);
  }
  return head + align16(pay);
}

/* Encodes the record of one chunk of n elements; the record is zero-padded. */
static int encode_record(int dt, const uint8_t *chunk, uint64_t n, const uint8_t *group_len,
                         int group_id, int coder, const pair_code *pc, uint8_t *rec, uint64_t cap,
                         uint64_t *rec_bytes, int *escape, zno_stats *st) {
  int nc = ncoded(dt), S = segsyms(dt);
  uint8_t *sym = (uint8_t *)malloc((size_t)n * 4 + 1);
  if (!sym) return ZNO_ERR_NOMEM;
  for (uint64_t i = 0; i < n; i++) {
    uint8_t s4[4];
    uint32_t raw;
    split_one(dt, load_elem(dt, chunk, i), s4, &raw);
    for (int p = 0; p < nc; p++) sym[(uint64_t)p * n + i] = s4[p];
  }
  stream_plan pl[4];
  uint64_t total = 0;
  if (escape) *escape = 0;
  for (int p = 0; p < nc; p++) {
    int rc = plan_stream(sym + (uint64_t)p * n, n, kbits(dt, p), S, p == 0 ? group_len : NULL,
                         group_id, p == 0 ? coder : ZNO_CODER_HUFFMAN, p == 0 ? pc : NULL, &pl[p], escape);
    if (rc < 0) {
      free(sym);
      return rc;
    }
    total += section_bytes_d(pl[p].mode, kbits(dt, p), n, pl[p].nseg, pl[p].bits, pl[p].d);
  }
  if (total > cap) {
    free(sym);
    return ZNO_ERR_CAPACITY;
  }
  memset(rec, 0, (size_t)total);
  uint64_t off = 0;
  for (int p = 0; p < nc; p++) {
    uint64_t sz = write_stream(rec + off, sym + (uint64_t)p * n, n, kbits(dt, p), &pl[p]);
    if (st) {
      st->mode_count[p][pl[p].mode]++;
      st->stream_bytes[p] += sz;
      st->payload_bits[p] += pl[p].mode == ZNO_RAW ? n * (uint64_t)kbits(dt, p) : pl[p].bits;
    }
    off += sz;
  }
  free(sym);
  *rec_bytes = total;
  return ZNO_OK;
}

int zno_encode_chunk2(int dt, const void *chunk, uint64_t n, const uint8_t *group_len, int group_id,
                      int coder, void *rec, uint64_t cap, uint64_t *rec_bytes, int *escape) {
  if (!valid_dtype(dt) || !rec_bytes || n == 0) return ZNO_ERR_ARG;
  if (coder != ZNO_CODER_HUFFMAN && (coder != ZNO_CODER_TANS || group_len)) return ZNO_ERR_ARG;
  return encode_record(dt, (const uint8_t *)chunk, n, group_len, group_id, coder, NULL, (uint8_t *)rec, cap,
                       rec_bytes, escape, NULL);
}
int zno_encode_chunk(int dt, const void *chunk, uint64_t n, const uint8_t *group_len, int group_id,
                     void *rec, uint64_t cap, uint64_t *rec_bytes, int *escape) {
  return zno_encode_chunk2(dt, chunk, n, group_len, group_id, ZNO_CODER_HUFFMAN, rec, cap, rec_bytes,
                           escape);
}

/* ------------------------------------------------------------------ */
/* NeuralZip-style tableset (R7)  [NZ Abstract]                        */
/* ------------------------------------------------------------------ */
struct zno_tableset {
  int dtype, K;
  uint32_t chunk_bytes, n_chunks;
  int n_tensors;
  uint64_t *n_elems;
  uint8_t (*len)[256]; /* [K][alphabet of stream 0] */
  uint8_t *map;        /* [n_chunks] group of each chunk */
  uint64_t cost[ROUNDS + 1];
  uint64_t hash;
  /* R9: packed exponent pairs (pairs = 1 when the setup was asked for them) */
  int pairs;
  uint8_t *packed;      /* [K] */
  uint8_t *nF;          /* [K] */
  uint8_t (*F)[16];     /* [K] the values of the pairs, by rank */
  uint8_t (*tlen)[512]; /* [K] token lengths: singles 0..255, pairs 256.. */
};

static void pair_code_of(const zno_tableset *ts, int g, pair_code *pc) {
  pc->nF = ts->nF[g];
  memcpy(pc->F, ts->F[g], 16);
  memset(pc->rank, 0xFF, 256);
  for (int i = 0; i < pc->nF; i++) pc->rank[pc->F[i]] = (uint8_t)i;
  pc->tlen = ts->tlen[g];
}


/* per group of a version-2 tableset: packing flag, |F|, F[16], 512 token
   lengths two per byte (even token in the low nibble) */
#define TS_PAIR_BYTES 274
static uint64_t ts_serial_bytes(const zno_tableset *ts) {
  int A = 1 << kbits(ts->dtype, 0);
  return 24 + 8 * (uint64_t)ts->n_tensors + (uint64_t)ts->K * (A / 2) + ts->n_chunks +
         (ts->pairs ? (uint64_t)ts->K * TS_PAIR_BYTES : 0);
}
static void ts_serialise(const zno_tableset *ts, uint8_t *b) {
  int A = 1 << kbits(ts->dtype, 0);
  put_u32(b, TS_MAGIC);
  put_u16(b + 4, ts->pairs ? 2 : VERSION);
  b[6] = (uint8_t)ts->dtype;
  b[7] = (uint8_t)ts->K;
  put_u32(b + 8, ts->chunk_bytes);
  put_u32(b + 12, (uint32_t)ts->n_tensors);
  put_u32(b + 16, ts->n_chunks);
  put_u32(b + 20, MAXLEN);
  uint8_t *q = b + 24;
  for (int t = 0; t < ts->n_tensors; t++, q += 8) put_u64(q, ts->n_elems[t]);
  for (int g = 0; g < ts->K; g++)
    for (int s = 0; s < A; s += 2) *q++ = (uint8_t)(ts->len[g][s] | (ts->len[g][s + 1] << 4));
  memcpy(q, ts->map, ts->n_chunks);
  q += ts->n_chunks;
  for (int g = 0; ts->pairs && g < ts->K; g++) {
    *q++ = ts->packed[g];
    *q++ = ts->nF[g];
    memcpy(q, ts->F[g], 16);
    q += 16;
    for (int t = 0; t < 512; t += 2) *q++ = (uint8_t)(ts->tlen[g][t] | (ts->tlen[g][t + 1] << 4));
  }
}
/* FNV-1a, 64-bit (Fowler, Noll, Vo). */
static uint64_t fnv1a64(const uint8_t *b, uint64_t n) {
  uint64_t h = 14695981039346656037ull;
  for (uint64_t i = 0; i < n; i++) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}
static int ts_rehash(zno_tableset *ts) {
  uint64_t n = ts_serial_bytes(ts);
  uint8_t *b = (uint8_t *)malloc((size_t)n);
  if (!b) return ZNO_ERR_NOMEM;
  ts_serialise(ts, b);
  ts->hash = fnv1a64(b, n);
  free(b);
  return ZNO_OK;
}

void zno_tableset_free(zno_tableset *ts) {
  if (!ts) return;
  free(ts->n_elems);
  free(ts->len);
  free(ts->map);
  free(ts->packed);
  free(ts->nF);
  free(ts->F);
  free(ts->tlen);
  free(ts);
}

static zno_tableset *ts_alloc(int dt, int K, uint32_t cb, int T, uint32_t M) {
  zno_tableset *ts = (zno_tableset *)calloc(1, sizeof *ts);
  if (!ts) return NULL;
  ts->dtype = dt;
  ts->K = K;
  ts->chunk_bytes = cb;
  ts->n_tensors = T;
  ts->n_chunks = M;
  ts->n_elems = (uint64_t *)calloc((size_t)T + 1, 8);
  ts->len = (uint8_t(*)[256])calloc((size_t)K + 1, 256);
  ts->map = (uint8_t *)calloc((size_t)M + 1, 1);
  ts->packed = (uint8_t *)calloc((size_t)K + 1, 1);
  ts->nF = (uint8_t *)calloc((size_t)K + 1, 1);
  ts->F = (uint8_t(*)[16])calloc((size_t)K + 1, 16);
  ts->tlen = (uint8_t(*)[512])calloc((size_t)K + 1, 512);
  if (!ts->n_elems || !ts->len || !ts->map || !ts->packed || !ts->nF || !ts->F || !ts->tlen) {
    zno_tableset_free(ts);
    return NULL;
  }
  return ts;
}

/* Coded size in bits of chunk histogram h under lengths len, or UINT64_MAX
 * if the table lacks a symbol the chunk uses. */
static uint64_t chunk_cost(const uint32_t *h, const uint8_t *len, int A) {
  uint64_t c = 0;
  for (int s = 0; s < A; s++) {
    if (!h[s]) continue;
    if (!len[s]) return UINT64_MAX;
    c += (uint64_t)h[s] * len[s];
  }
  return c;
}

static int tables_from_assignment(const uint32_t *hist, uint32_t M, int A, int K,
                                  const uint8_t *map, uint8_t (*len)[256]) {
  uint64_t *H = (uint64_t *)calloc((size_t)K * A, 8);
  if (!H) return ZNO_ERR_NOMEM;
  for (uint32_t c = 0; c < M; c++)
    for (int s = 0; s < A; s++) H[(uint64_t)map[c] * A + s] += hist[(uint64_t)c * A + s];
  for (int g = 0; g < K; g++) {
    int rc = zno_group_lengths(H + (uint64_t)g * A, A, MAXLEN, len[g]);
    if (rc < 0) {
      free(H);
      return rc;
    }
  }
  free(H);
  return ZNO_OK;
}

static uint64_t total_cost(const uint32_t *hist, uint32_t M, int A, const uint8_t *map,
                           uint8_t (*len)[256]) {
  uint64_t t = 0;
  for (uint32_t c = 0; c < M; c++) t += chunk_cost(hist + (uint64_t)c * A, len[map[c]], A);
  return t;
}

/* Exponent-stream (stream 0) histogram of every chunk of every tensor, in
 * tensor order then chunk order; cn[c] = the chunk's element count. */
static void chunk_histograms(int dt, const void *const *tensors, const uint64_t *n_elems, int T,
                             uint32_t cb, uint32_t *hist, uint64_t *cn) {
  const int A = 1 << kbits(dt, 0);
  const uint64_t ce = chunk_elems(dt, cb);
  uint32_t c = 0;
  for (int t = 0; t < T; t++) {
    const uint8_t *b = (const uint8_t *)tensors[t];
    for (uint64_t i0 = 0; i0 < n_elems[t]; i0 += ce, c++) {
      uint64_t n = n_elems[t] - i0 < ce ? n_elems[t] - i0 : ce;
      cn[c] = n;
      for (uint64_t i = 0; i < n; i++) {
        uint8_t s4[4];
        uint32_t raw;
        split_one(dt, load_elem(dt, b, i0 + i), s4, &raw);
        hist[(uint64_t)c * A + s4[0]]++;
      }
    }
  }
}

typedef struct {
  uint64_t key;
  uint32_t c;
} keyed;
static int cmp_keyed(const void *a, const void *b) {
  const keyed *x = (const keyed *)a, *y = (const keyed *)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return x->c < y->c ? -1 : x->c > y->c;
}

/* R9: every group's pair code, from the final assignment (hist: the chunks'
 * exponent histograms). */
static int setup_pairs(zno_tableset *ts, const uint32_t *hist, const void *const *tensors,
                       const uint64_t *n_elems, int T) {
  const int K = ts->K, dt = ts->dtype;
  const uint32_t M = ts->n_chunks;
  const uint64_t ce = chunk_elems(dt, ts->chunk_bytes);
  uint64_t *H = (uint64_t *)calloc((size_t)K * 256, 8), *Tk = (uint64_t *)calloc((size_t)K * 512, 8);
  uint8_t *sym = (uint8_t *)malloc((size_t)ce);
  pair_code *pc = (pair_code *)calloc((size_t)K, sizeof(pair_code));
  if (!H || !Tk || !sym || !pc) {
    free(H), free(Tk), free(sym), free(pc);
    return ZNO_ERR_NOMEM;
  }
  for (uint32_t c = 0; c < M; c++)
    for (int s = 0; s < 256; s++) H[(uint64_t)ts->map[c] * 256 + s] += hist[(uint64_t)c * 256 + s];
  /* F: the values of largest pooled count, ties to the smaller value */
  for (int g = 0; g < K; g++) {
    uint8_t taken[256] = {0};
    int nF = 0;
    for (; nF < 16; nF++) {
      int best = -1;
      for (int s = 0; s < 256; s++)
        if (!taken[s] && H[(uint64_t)g * 256 + s] && (best < 0 || H[(uint64_t)g * 256 + s] > H[(uint64_t)g * 256 + best]))
          best = s;
      if (best < 0) break;
      taken[best] = 1;
      ts->F[g][nF] = (uint8_t)best;
    }
    ts->nF[g] = (uint8_t)nF;
    pair_code_of(ts, g, &pc[g]);
  }
  /* token counts over the group's chunks */
  uint32_t c = 0;
  for (int t = 0; t < T; t++) {
    const uint8_t *b = (const uint8_t *)tensors[t];
    for (uint64_t i0 = 0; i0 < n_elems[t]; i0 += ce, c++) {
      const uint64_t n = n_elems[t] - i0 < ce ? n_elems[t] - i0 : ce;
      const int g = ts->map[c];
      for (uint64_t i = 0; i < n; i++) {
        uint8_t s4[4];
        uint32_t raw;
        split_one(dt, load_elem(dt, b, i0 + i), s4, &raw);
        sym[i] = s4[0];
      }
      uint64_t *tk = Tk + (uint64_t)g * 512;
      for (uint64_t a = 0; a < n; a += STRIP) {
        const uint64_t e = a + STRIP < n ? a + STRIP : n;
        for (uint64_t i = a; i < e; i += 2) {
          const int rx = pc[g].rank[sym[i]], ry = i + 1 < e ? pc[g].rank[sym[i + 1]] : 0xFF;
          if (i + 1 < e && rx < pc[g].nF && ry < pc[g].nF) {
            tk[256 + 16 * rx + ry]++;
          } else {
            tk[sym[i]]++;
            if (i + 1 < e) tk[sym[i + 1]]++;
          }
        }
      }
    }
  }
  int rc = ZNO_OK;
  for (int g = 0; g < K && rc == ZNO_OK; g++) {
    rc = zno_group_lengths(Tk + (uint64_t)g * 512, 512, MAXLEN, ts->tlen[g]);
    if (rc < 0) break;
    rc = ZNO_OK;
    uint64_t bt = 0, bs = 0;
    for (int t = 0; t < 512; t++) bt += Tk[(uint64_t)g * 512 + t] * ts->tlen[g][t];
    for (int s = 0; s < 256; s++) bs += H[(uint64_t)g * 256 + s] * ts->len[g][s];
    ts->packed[g] = bt < bs;
  }
  ts->pairs = 1;
  free(H), free(Tk), free(sym), free(pc);
  return rc;
}

int zno_setup(int dt, const void *const *tensors, const uint64_t *n_elems, int T, uint32_t cb,
              int K, zno_tableset **out) {
  return zno_setup2(dt, tensors, n_elems, T, cb, K, 0, out);
}

int zno_setup2(int dt, const void *const *tensors, const uint64_t *n_elems, int T, uint32_t cb,
               int K, int flags, zno_tableset **out) {
  if (!out || !valid_dtype(dt) || !valid_chunk(cb) || T < 1 || K < 0 || K > 255) return ZNO_ERR_ARG;
  if ((flags & ~ZNO_SETUP_PAIRS) || ((flags & ZNO_SETUP_PAIRS) && (dt != ZNO_BF16 || K < 1)))
    return ZNO_ERR_ARG;
  uint32_t M = 0;
  for (int t = 0; t < T; t++) M += (uint32_t)nchunks_of(dt, n_elems[t], cb);
  zno_tableset *ts = ts_alloc(dt, K, cb, T, M);
  if (!ts) return ZNO_ERR_NOMEM;
  memcpy(ts->n_elems, n_elems, 8 * (size_t)T);
  if (K == 0) {
    int rc = ts_rehash(ts);
    if (rc < 0) {
      zno_tableset_free(ts);
      return rc;
    }
    *out = ts;
    return ZNO_OK;
  }
  if (!tensors) {
    zno_tableset_free(ts);
    return ZNO_ERR_ARG;
  }
  int A = 1 << kbits(dt, 0);
  uint32_t *hist = (uint32_t *)calloc((size_t)M * A + 1, 4);
  uint64_t *cn = (uint64_t *)calloc((size_t)M + 1, 8);
  keyed *keys = (keyed *)calloc((size_t)M + 1, sizeof(keyed));
  if (!hist || !cn || !keys) {
    free(hist), free(cn), free(keys), zno_tableset_free(ts);
    return ZNO_ERR_NOMEM;
  }
  /* (1) exponent-stream histogram of every chunk of every tensor */
  chunk_histograms(dt, tensors, n_elems, T, cb, hist, cn);
  uint32_t c;
  /* (2) initial groups: chunks ordered by their mean exponent, cut evenly */
  for (c = 0; c < M; c++) {
    uint64_t sum = 0;
    for (int s = 0; s < A; s++) sum += (uint64_t)s * hist[(uint64_t)c * A + s];
    keys[c].key = (sum << 16) / cn[c];
    keys[c].c = c;
  }
  qsort(keys, M, sizeof(keyed), cmp_keyed);
  for (int g = 0; g < K; g++) {
    uint64_t lo = (uint64_t)M * g / K, hi = (uint64_t)M * (g + 1) / K;
    for (uint64_t i = lo; i < hi; i++) ts->map[keys[i].c] = (uint8_t)g;
  }
  /* (3) rounds: tables from the current groups, then reassignment */
  int rc = ZNO_OK;
  for (int r = 0; r < ROUNDS && rc == ZNO_OK; r++) {
    rc = tables_from_assignment(hist, M, A, K, ts->map, ts->len);
    if (rc < 0) break;
    ts->cost[r] = total_cost(hist, M, A, ts->map, ts->len);
    for (c = 0; c < M; c++) {
      uint64_t best = UINT64_MAX;
      int bg = ts->map[c];
      for (int g = 0; g < K; g++) {
        uint64_t x = chunk_cost(hist + (uint64_t)c * A, ts->len[g], A);
        if (x < best) { /* strict: ties keep the smaller group id */
          best = x;
          bg = g;
        }
      }
      ts->map[c] = (uint8_t)bg;
    }
  }
  /* (4) final tables from the final assignment */
  if (rc == ZNO_OK) rc = tables_from_assignment(hist, M, A, K, ts->map, ts->len);
  if (rc == ZNO_OK) ts->cost[ROUNDS] = total_cost(hist, M, A, ts->map, ts->len);
  /* (5) R9: pair codes */
  if (rc == ZNO_OK && (flags & ZNO_SETUP_PAIRS)) rc = setup_pairs(ts, hist, tensors, n_elems, T);
  free(hist), free(cn), free(keys);
  if (rc == ZNO_OK) rc = ts_rehash(ts);
  if (rc < 0) {
    zno_tableset_free(ts);
    return rc;
  }
  *out = ts;
  return ZNO_OK;
}

/* Transfer of a setup to other tensors of the same dtype (another model
 * architecture of the same kind  [NZ Abstract]): the source's K group codes are
 * kept as they are; every chunk of the new tensors goes to the group code
 * that codes its exponent histogram in the fewest bits, ties to the smaller
 * group id; a chunk that every group code lacks a symbol for goes to group 0
 * (compression then codes it with its own table).  The assignment depends on
 * the chunk's content only, not on its position.  The cost history is the
 * source's (the tables were fit there). */
int zno_setup_transfer(const zno_tableset *src, const void *const *tensors, const uint64_t *n_elems,
                       int T, zno_tableset **out) {
  if (!out) return ZNO_ERR_ARG;
  *out = NULL;
  if (!src || src->K < 1 || !tensors || !n_elems || T < 1) return ZNO_ERR_ARG;
  const int dt = src->dtype, K = src->K, A = 1 << kbits(dt, 0);
  const uint32_t cb = src->chunk_bytes;
  uint64_t M64 = 0;
  for (int t = 0; t < T; t++) {
    if (n_elems[t] && !tensors[t]) return ZNO_ERR_ARG;
    M64 += nchunks_of(dt, n_elems[t], cb);
  }
  if (M64 > 0xFFFFFFFFull) return ZNO_ERR_ARG;
  const uint32_t M = (uint32_t)M64;
  zno_tableset *ts = ts_alloc(dt, K, cb, T, M);
  if (!ts) return ZNO_ERR_NOMEM;
  memcpy(ts->n_elems, n_elems, 8 * (size_t)T);
  memcpy(ts->len, src->len, (size_t)K * 256);
  memcpy(ts->cost, src->cost, sizeof ts->cost);
  ts->pairs = src->pairs;
  memcpy(ts->packed, src->packed, (size_t)K);
  memcpy(ts->nF, src->nF, (size_t)K);
  memcpy(ts->F, src->F, (size_t)K * 16);
  memcpy(ts->tlen, src->tlen, (size_t)K * 512);
  uint32_t *hist = (uint32_t *)calloc((size_t)M * A + 1, 4);
  uint64_t *cn = (uint64_t *)calloc((size_t)M + 1, 8);
  if (!hist || !cn) {
    free(hist), free(cn), zno_tableset_free(ts);
    return ZNO_ERR_NOMEM;
  }
  chunk_histograms(dt, tensors, n_elems, T, cb, hist, cn);
  for (uint32_t c = 0; c < M; c++) {
    uint64_t best = UINT64_MAX;
    int bg = 0;
    for (int g = 0; g < K; g++) {
      uint64_t x = chunk_cost(hist + (uint64_t)c * A, ts->len[g], A);
      if (x < best) { /* strict: ties keep the smaller group id */
        best = x;
        bg = g;
      }
    }
    ts->map[c] = (uint8_t)bg;
  }
  free(hist), free(cn);
  int rc = ts_rehash(ts);
  if (rc < 0) {
    zno_tableset_free(ts);
    return rc;
  }
  *out = ts;
  return ZNO_OK;
}

int zno_tableset_info(const zno_tableset *ts, int *K, uint32_t *n_chunks, uint64_t *hash) {
  if (!ts) return ZNO_ERR_ARG;
  if (K) *K = ts->K;
  if (n_chunks) *n_chunks = ts->n_chunks;
  if (hash) *hash = ts->hash;
  return ZNO_OK;
}
int zno_tableset_lengths(const zno_tableset *ts, int g, uint8_t *len) {
  if (!ts || g < 0 || g >= ts->K) return ZNO_ERR_ARG;
  memcpy(len, ts->len[g], (size_t)(1 << kbits(ts->dtype, 0)));
  return ZNO_OK;
}
int zno_tableset_map(const zno_tableset *ts, uint8_t *map) {
  if (!ts) return ZNO_ERR_ARG;
  memcpy(map, ts->map, ts->n_chunks);
  return ZNO_OK;
}
int zno_tableset_cost_history(const zno_tableset *ts, uint64_t *cost) {
  if (!ts) return ZNO_ERR_ARG;
  memcpy(cost, ts->cost, sizeof ts->cost);
  return ZNO_OK;
}
int zno_tableset_pairs(const zno_tableset *ts, int g, int *packed, int *nF, uint8_t *F, uint8_t *tlen) {
  if (!ts || g < 0 || g >= ts->K) return ZNO_ERR_ARG;
  if (packed) *packed = ts->pairs ? ts->packed[g] : 0;
  if (nF) *nF = ts->pairs ? ts->nF[g] : 0;
  if (F) memcpy(F, ts->F[g], 16);
  if (tlen) memcpy(tlen, ts->tlen[g], 512);
  return ts->pairs;
}
int zno_tableset_save(const zno_tableset *ts, void *buf, uint64_t cap, uint64_t *len) {
  if (!ts || !len) return ZNO_ERR_ARG;
  *len = ts_serial_bytes(ts);
  if (!buf) return ZNO_OK;
  if (cap < *len) return ZNO_ERR_CAPACITY;
  ts_serialise(ts, (uint8_t *)buf);
  return ZNO_OK;
}
int zno_tableset_load(const void *buf, uint64_t len, zno_tableset **out) {
  const uint8_t *b = (const uint8_t *)buf;
  if (!b || !out || len < 24 || get_u32(b) != TS_MAGIC || get_u32(b + 20) != MAXLEN) return ZNO_ERR_CORRUPT;
  /* version 2: with the pair codes of R9 (BF16 with groups only) */
  const int ver = (int)get_u16(b + 4);
  int dt = b[6], K = b[7], T = (int)get_u32(b + 12);
  uint32_t cb = get_u32(b + 8), M = get_u32(b + 16);
  if ((ver != VERSION && ver != 2) || !valid_dtype(dt) || !valid_chunk(cb) || T < 1) return ZNO_ERR_CORRUPT;
  const int pairs = ver == 2;
  if (pairs && (dt != ZNO_BF16 || K < 1)) return ZNO_ERR_CORRUPT;
  int A = 1 << kbits(dt, 0);
  if (len != 24 + 8 * (uint64_t)T + (uint64_t)K * (A / 2) + M + (pairs ? (uint64_t)K * TS_PAIR_BYTES : 0))
    return ZNO_ERR_CORRUPT;
  zno_tableset *ts = ts_alloc(dt, K, cb, T, M);
  if (!ts) return ZNO_ERR_NOMEM;
  const uint8_t *q = b + 24;
  uint64_t msum = 0;
  for (int t = 0; t < T; t++, q += 8) {
    ts->n_elems[t] = get_u64(q);
    msum += nchunks_of(dt, ts->n_elems[t], cb);
  }
  for (int g = 0; g < K; g++)
    for (int s = 0; s < A; s += 2, q++) {
      ts->len[g][s] = *q & 15;
      ts->len[g][s + 1] = *q >> 4;
    }
  memcpy(ts->map, q, M);
  q += M;
  int bad = msum != M;
  ts->pairs = pairs;
  for (int g = 0; pairs && g < K; g++) {
    ts->packed[g] = q[0];
    ts->nF[g] = q[1];
    memcpy(ts->F[g], q + 2, 16);
    for (int t = 0; t < 512; t += 2) {
      ts->tlen[g][t] = q[18 + t / 2] & 15;
      ts->tlen[g][t + 1] = q[18 + t / 2] >> 4;
    }
    q += TS_PAIR_BYTES;
    /* a flag, at most 16 distinct values of F (zero past |F|), lengths within
       the limit, no pair token past |F|, and a packing group's token code
       complete (Kraft equality) */
    const int nF = ts->nF[g];
    bad |= ts->packed[g] > 1 || nF > 16;
    uint8_t seen[256] = {0};
    for (int i = 0; i < 16 && !bad; i++) {
      if (i < nF) bad |= seen[ts->F[g][i]]++ != 0;
      else bad |= ts->F[g][i] != 0;
    }
    uint64_t kraft = 0;
    int d = 0;
    for (int t = 0; t < 512 && !bad; t++) {
      const int l = ts->tlen[g][t];
      bad |= l > MAXLEN;
      if (t >= 256 && (((t - 256) >> 4) >= nF || ((t - 256) & 15) >= nF)) bad |= l != 0;
      if (l && l <= MAXLEN) {
        kraft += (uint64_t)1 << (MAXLEN - l);
        d++;
      }
    }
    if (ts->packed[g] && !bad) bad = d < 2 || kraft != ((uint64_t)1 << MAXLEN);
  }
  /* a plan without groups stores its map as zero bytes; with groups each
     byte names one of the K groups */
  for (uint32_t c = 0; c < M && !bad; c++) bad = K ? ts->map[c] >= K : ts->map[c] != 0;
  for (int g = 0; g < K && !bad; g++)
    for (int s = 0; s < A; s++) bad |= ts->len[g][s] > MAXLEN;
  if (bad || ts_rehash(ts) < 0) {
    zno_tableset_free(ts);
    return ZNO_ERR_CORRUPT;
  }
  *out = ts;
  return ZNO_OK;
}

/* ------------------------------------------------------------------ */
/* R6: container                                                       */
/* ------------------------------------------------------------------ */
typedef struct {
  uint64_t off_dir, off_records;
  uint64_t n_chunks;
} layout;

static void make_layout(int dt, const uint64_t *n, int T, uint32_t cb, uint64_t *raw_off,
                        layout *lo) {
  uint64_t M = 0;
  for (int t = 0; t < T; t++) M += nchunks_of(dt, n[t], cb);
  lo->n_chunks = M;
  lo->off_dir = 64 + 16 * (uint64_t)T;
  uint64_t cur = align16(lo->off_dir + 8 * ((uint64_t)M + 1));
  for (int t = 0; t < T; t++) {
    raw_off[t] = cur;
    cur = align16(cur + rawplane_bytes(dt, n[t]));
  }
  lo->off_records = cur;
}

int zno_compress_bound(int dt, const uint64_t *n, int T, uint32_t cb, uint64_t *bound) {
  if (!valid_dtype(dt) || !valid_chunk(cb) || T < 1 || !n || !bound) return ZNO_ERR_ARG;
  uint64_t *raw_off = (uint64_t *)calloc((size_t)T, 8);
  if (!raw_off) return ZNO_ERR_NOMEM;
  layout lo;
  make_layout(dt, n, T, cb, raw_off, &lo);
  free(raw_off);
  uint64_t b = lo.off_records + 16, ce = chunk_elems(dt, cb);
  for (int t = 0; t < T; t++)
    for (uint64_t i0 = 0; i0 < n[t]; i0 += ce) {
      uint64_t m = n[t] - i0 < ce ? n[t] - i0 : ce;
      for (int p = 0; p < ncoded(dt); p++) b += section_bytes(ZNO_RAW, kbits(dt, p), m, 0, 0);
    }
  *bound = b;
  return ZNO_OK;
}

static int ts_matches(const zno_tableset *ts, int dt, const uint64_t *n, int T, uint32_t cb) {
  if (ts->dtype != dt || ts->chunk_bytes != cb || ts->n_tensors != T) return 0;
  for (int t = 0; t < T; t++)
    if (ts->n_elems[t] != n[t]) return 0;
  return 1;
}

int zno_compress(int dt, const void *const *tensors, const uint64_t *n, int T, uint32_t cb,
                 const zno_tableset *ts, void *outv, uint64_t cap, uint64_t *out_bytes,
                 zno_stats *st) {
  return zno_compress2(dt, tensors, n, T, cb, ts, ZNO_CODER_HUFFMAN, outv, cap, out_bytes, st);
}

int zno_compress2(int dt, const void *const *tensors, const uint64_t *n, int T, uint32_t cb,
                  const zno_tableset *ts, int coder, void *outv, uint64_t cap, uint64_t *out_bytes,
                  zno_stats *st) {
  if (!valid_dtype(dt) || !valid_chunk(cb) || T < 1 || !n || !outv || !out_bytes) return ZNO_ERR_ARG;
  if (coder != ZNO_CODER_HUFFMAN && (coder != ZNO_CODER_TANS || (ts && ts->K > 0))) return ZNO_ERR_ARG;
  for (int t = 0; t < T; t++)
    if (n[t] && (!tensors || !tensors[t])) return ZNO_ERR_ARG;
  int grouped = ts && ts->K > 0;
  if (grouped && !ts_matches(ts, dt, n, T, cb)) return ZNO_ERR_TABLESET;
  uint8_t *out = (uint8_t *)outv;
  uint64_t *raw_off = (uint64_t *)calloc((size_t)T, 8);
  if (!raw_off) return ZNO_ERR_NOMEM;
  layout lo;
  make_layout(dt, n, T, cb, raw_off, &lo);
  if (lo.n_chunks > 0xFFFFFFFFull) {
    free(raw_off);
    return ZNO_ERR_ARG;
  }
  if (lo.off_records + 16 > cap) {
    free(raw_off);
    return ZNO_ERR_CAPACITY;
  }
  if (st) memset(st, 0, sizeof *st);
  memset(out, 0, (size_t)lo.off_records);
  uint64_t ntot = 0;
  for (int t = 0; t < T; t++) ntot += n[t];
  /* header */
  put_u32(out, MAGIC);
  put_u16(out + 4, VERSION);
  out[6] = (uint8_t)dt;
  out[7] = grouped ? 1 : 0;
  put_u32(out + 8, (uint32_t)T);
  put_u32(out + 12, cb);
  put_u64(out + 16, ntot);
  put_u32(out + 24, (uint32_t)lo.n_chunks);
  put_u16(out + 28, (uint32_t)segsyms(dt));
  out[30] = MAXLEN;
  out[31] = (uint8_t)ncoded(dt);
  put_u64(out + 32, grouped ? ts->hash : 0);
  put_u64(out + 40, lo.off_dir);
  put_u64(out + 48, lo.off_records);
  /* tensor table and always-raw sections */
  for (int t = 0; t < T; t++) {
    put_u64(out + 64 + 16 * (uint64_t)t, n[t]);
    put_u64(out + 72 + 16 * (uint64_t)t, raw_off[t]);
    const uint8_t *b = (const uint8_t *)tensors[t];
    for (uint64_t i = 0; i < n[t]; i++) {
      uint8_t s4[4];
      uint32_t raw;
      split_one(dt, load_elem(dt, b, i), s4, &raw);
      if (dt == ZNO_BF16) out[raw_off[t] + i] = (uint8_t)raw;
      if (dt == ZNO_FP8_E4M3 && raw) out[raw_off[t] + i / 8] |= (uint8_t)(1u << (i % 8));
      if (dt == ZNO_FP4X2_E2M1 && raw) out[raw_off[t] + i / 4] |= (uint8_t)(raw << (2 * (i % 4)));
    }
    if (st) st->raw_plane_bytes += rawplane_bytes(dt, n[t]);
  }
  /* records */
  uint64_t pos = lo.off_records, ce = chunk_elems(dt, cb);
  uint32_t c = 0;
  int rc = ZNO_OK;
  for (int t = 0; t < T && rc == ZNO_OK; t++) {
    const uint8_t *b = (const uint8_t *)tensors[t];
    for (uint64_t i0 = 0; i0 < n[t]; i0 += ce, c++) {
      uint64_t m = n[t] - i0 < ce ? n[t] - i0 : ce, sz = 0;
      int esc = 0, g = grouped ? ts->map[c] : 0;
      put_u64(out + lo.off_dir + 8 * (uint64_t)c, pos);
      if (pos > cap) {
        rc = ZNO_ERR_CAPACITY;
        break;
      }
      pair_code pcg;
      const int packed = grouped && ts->pairs && ts->packed[g];
      if (packed) pair_code_of(ts, g, &pcg);
      rc = encode_record(dt, b + i0 * (uint64_t)esize(dt), m, grouped ? ts->len[g] : NULL, g, coder,
                         packed ? &pcg : NULL, out + pos, cap - pos, &sz, &esc, st);
      if (rc < 0) break;
      if (st) st->escapes += (uint64_t)esc;
      pos += sz;
    }
  }
  free(raw_off);
  if (rc < 0) return rc;
  if (pos + 16 > cap) return ZNO_ERR_CAPACITY;
  put_u64(out + lo.off_dir + 8 * (uint64_t)lo.n_chunks, pos);
  memset(out + pos, 0, 16);
  put_u64(out + 56, pos + 16);
  *out_bytes = pos + 16;
  return ZNO_OK;
}

/* ------------------------------------------------------------------ */
/* C10: decoding, with every structural check                          */
/* ------------------------------------------------------------------ */
int zno_header(const void *inv, uint64_t in_bytes, int *dt, int *T, uint64_t *ntot, uint32_t *cb,
               uint32_t *nchunks, uint64_t *total, uint64_t *hash) {
  const uint8_t *in = (const uint8_t *)inv;
  if (!in || in_bytes < 64) return ZNO_ERR_CORRUPT;
  if (get_u32(in) != MAGIC || get_u16(in + 4) != VERSION) return ZNO_ERR_CORRUPT;
  if (!valid_dtype(in[6]) || (in[7] & ~1u) || in[30] != MAXLEN || in[31] != ncoded(in[6]) ||
      get_u16(in + 28) != (uint32_t)segsyms(in[6]) || !valid_chunk(get_u32(in + 12)))
    return ZNO_ERR_CORRUPT;
  /* R6: a container holds at least one tensor, and its hash field is zero
     unless the group bit is set */
  if (get_u32(in + 8) < 1 || (!(in[7] & 1) && get_u64(in + 32) != 0)) return ZNO_ERR_CORRUPT;
  if (dt) *dt = in[6];
  if (T) *T = (int)get_u32(in + 8);
  if (ntot) *ntot = get_u64(in + 16);
  if (cb) *cb = get_u32(in + 12);
  if (nchunks) *nchunks = get_u32(in + 24);
  if (total) *total = get_u64(in + 56);
  if (hash) *hash = get_u64(in + 32);
  return ZNO_OK;
}

/* R9: the tokens of a GROUP section whose group packs pairs; q: the segment
 * lengths.  Returns the section size, or a negative status. */
static int64_t decode_pairs(const uint8_t *q, const uint8_t *payload, uint64_t pay, uint64_t head,
                            uint64_t n, int nseg, const zno_tableset *ts, int g, uint8_t *sym) {
  const uint8_t *tlen = ts->tlen[g];
  uint64_t kraft = 0;
  int count[17] = {0}, d = 0;
  for (int t = 0; t < 512; t++) {
    if (tlen[t] > MAXLEN) return ZNO_ERR_CORRUPT;
    if (tlen[t]) {
      kraft += (uint64_t)1 << (MAXLEN - tlen[t]);
      count[tlen[t]]++;
      d++;
    }
  }
  if (d < 2 || kraft != ((uint64_t)1 << MAXLEN)) return ZNO_ERR_CORRUPT;
  int sorted[512], offs[17], first[17], o = 0;
  uint32_t code = 0;
  for (int l = 1; l <= MAXLEN; l++) {
    offs[l] = o;
    o += count[l];
  }
  {
    int fill[17];
    memcpy(fill, offs, sizeof fill);
    for (int t = 0; t < 512; t++)
      if (tlen[t]) sorted[fill[tlen[t]]++] = t;
  }
  for (int l = 1; l <= MAXLEN; l++) {
    code = (code + (uint32_t)count[l - 1]) << 1;
    first[l] = (int)code;
  }
  uint64_t total_bits = 0;
  for (int j = 0; j < nseg; j++) total_bits += get_u16(q + 2 * j);
  if (pay != 4 * ((total_bits + 31) / 32)) return ZNO_ERR_CORRUPT;
  uint64_t seg_start = 0;
  for (int j = 0; j < nseg; j++) {
    uint64_t sb = get_u16(q + 2 * j);
    bitr br = {payload, seg_start, seg_start + sb};
    /* the segment's positions: strips j, j + nseg, ...; a pair fills two */
    uint64_t i = (uint64_t)j * STRIP;
    int half = 0;   /* 1: the next position takes a pair's second value */
    uint8_t second = 0;
    while (i < n) {
      if (half) {
        sym[i] = second;
        half = 0;
      } else {
        int c = 0, found = -1;
        for (int l = 1; l <= MAXLEN; l++) {
          unsigned bit;
          if (get_bit(&br, &bit)) return ZNO_ERR_CORRUPT;
          c = (c << 1) | (int)bit;
          if (c >= first[l] && c - first[l] < count[l]) {
            found = sorted[offs[l] + c - first[l]];
            break;
          }
        }
        if (found < 0) return ZNO_ERR_CORRUPT;
        if (found < 256) {
          sym[i] = (uint8_t)found;
        } else {
          sym[i] = ts->F[g][(found - 256) >> 4];
          second = ts->F[g][(found - 256) & 15];
          half = 1;
        }
      }
      i = ((i + 1) % STRIP) ? i + 1 : i + 1 + (uint64_t)(nseg - 1) * STRIP;
    }
    if (half) return ZNO_ERR_CORRUPT;             /* a pair past the segment's last value */
    if (br.pos != br.end) return ZNO_ERR_CORRUPT; /* segment length must be exact */
    seg_start += sb;
  }
  return (int64_t)(head + align16(pay));
}

/* Decodes one stream section of n symbols at sec (within [sec, lim)).
 * Returns the section size, or a negative status. */
static int64_t decode_stream(const uint8_t *sec, const uint8_t *lim, uint64_t n, int k, int S,
                             const zno_tableset *ts, int allow_group, int allow_tans, uint8_t *sym) {
  int A = 1 << k;
  if (lim - sec < 16) return ZNO_ERR_CORRUPT;
  int mode = sec[0], aux = sec[1], nseg = (int)get_u16(sec + 2);
  uint64_t pay = get_u32(sec + 4);
  int want_seg = (int)((n + (uint64_t)S - 1) / (uint64_t)S);
  if (mode > ZNO_TANS || nseg != want_seg) return ZNO_ERR_CORRUPT;
  /* R8: tANS codes the exponent stream (the first coded stream) only */
  if (mode == ZNO_TANS && !allow_tans) return ZNO_ERR_CORRUPT;
  int dpresent = 0;
  if (mode == ZNO_TANS) {
    if (lim - sec < 8 + A / 8) return ZNO_ERR_CORRUPT;
    for (int s = 0; s < A; s++) dpresent += (sec[8 + s / 8] >> (s % 8)) & 1;
  }
  uint64_t head = head_bytes_d(mode, k, nseg, dpresent);
  if ((uint64_t)(lim - sec) < head + align16(pay)) return ZNO_ERR_CORRUPT;
  const uint8_t *payload = sec + head;
  if (mode == ZNO_TANS) {
    /* R8: counts of the present symbols summing to 2^11, each at least 1,
       then each segment from its final state */
    if (aux != 0) return ZNO_ERR_CORRUPT;
    uint32_t q[256];
    uint64_t sum = 0;
    const uint8_t *qp = sec + 8 + A / 8;
    for (int s = 0; s < A; s++) {
      q[s] = 0;
      if ((sec[8 + s / 8] >> (s % 8)) & 1) {
        q[s] = get_u16(qp);
        qp += 2;
        if (q[s] == 0) return ZNO_ERR_CORRUPT;
      }
      sum += q[s];
    }
    if (sum != TL) return ZNO_ERR_CORRUPT;
    const uint8_t *sbits = qp;
    uint64_t total_bits = 0;
    for (int j = 0; j < nseg; j++) total_bits += get_u16(sbits + 2 * j);
    if (pay != 4 * ((total_bits + 31) / 32)) return ZNO_ERR_CORRUPT;
    uint8_t spread[TL];
    uint32_t rank[TL];
    zno_tans_spread(q, A, spread);
    tans_ranks(spread, rank);
    uint8_t *seg = (uint8_t *)malloc((size_t)n);
    if (!seg) return ZNO_ERR_NOMEM;
    uint64_t seg_start = 0;
    for (int j = 0; j < nseg; j++) {
      uint64_t sb = get_u16(sbits + 2 * j);
      bitr br = {payload, seg_start, seg_start + sb};
      uint32_t st = 0;
      for (int b = 0; b < ZNO_TANS_LOG; b++) {
        unsigned bit;
        if (get_bit(&br, &bit)) {
          free(seg);
          return ZNO_ERR_CORRUPT;
        }
        st |= (uint32_t)bit << b;
      }
      /* the segment's symbols: strips j, j + nseg, ... */
      uint64_t m = 0;
      for (uint64_t q0 = (uint64_t)j * STRIP; q0 < n; q0 += (uint64_t)nseg * STRIP)
        for (uint64_t i = q0; i < n && i < q0 + STRIP; i++) m++;
      if (tans_decode_segment(q, spread, rank, &br, st, m, seg, 0) < 0) {
        free(seg);
        return ZNO_ERR_CORRUPT;
      }
      m = 0;
      for (uint64_t q0 = (uint64_t)j * STRIP; q0 < n; q0 += (uint64_t)nseg * STRIP)
        for (uint64_t i = q0; i < n && i < q0 + STRIP; i++) sym[i] = seg[m++];
      seg_start += sb;
    }
    free(seg);
    return (int64_t)(head + align16(pay));
  }
  if (mode == ZNO_CONST) {
    if (aux >= A || pay != 0) return ZNO_ERR_CORRUPT;
    for (uint64_t i = 0; i < n; i++) sym[i] = (uint8_t)aux;
    return (int64_t)head;
  }
  if (mode == ZNO_RAW) {
    if (aux != 0 || pay != (n * (uint64_t)k + 7) / 8) return ZNO_ERR_CORRUPT;
    bitr br = {payload, 0, pay * 8};
    for (uint64_t i = 0; i < n; i++) {
      unsigned v = 0, bit;
      for (int q = 0; q < k; q++) {
        if (get_bit(&br, &bit)) return ZNO_ERR_CORRUPT;
        v |= bit << q;
      }
      sym[i] = (uint8_t)v;
    }
    return (int64_t)(head + align16(pay));
  }
  /* HUFF or GROUP: lengths, then canonical decoding bit by bit */
  uint8_t len[256];
  const uint8_t *q = sec + 8;
  if (mode == ZNO_HUFF) {
    if (aux != 0) return ZNO_ERR_CORRUPT;
    for (int s = 0; s < A; s += 2) {
      len[s] = q[s / 2] & 15;
      len[s + 1] = q[s / 2] >> 4;
    }
    q += A / 2;
  } else {
    if (!allow_group) return ZNO_ERR_CORRUPT;
    if (!ts || ts->K == 0 || aux >= ts->K) return ZNO_ERR_TABLESET;
    if (ts->pairs && ts->packed[aux]) return decode_pairs(q, payload, pay, head, n, nseg, ts, aux, sym);
    memcpy(len, ts->len[aux], (size_t)A);
  }
  /* the lengths must form a complete prefix code (Kraft equality) */
  uint64_t kraft = 0;
  int count[17] = {0}, d = 0;
  for (int s = 0; s < A; s++) {
    if (len[s] > MAXLEN) return ZNO_ERR_CORRUPT;
    if (len[s]) {
      kraft += (uint64_t)1 << (MAXLEN - len[s]);
      count[len[s]]++;
      d++;
    }
  }
  if (d < 2 || kraft != ((uint64_t)1 << MAXLEN)) return ZNO_ERR_CORRUPT;
  /* symbols sorted by (length, symbol); first code of each length */
  int sorted[256], offs[17], first[17], o = 0;
  uint32_t code = 0;
  for (int l = 1; l <= MAXLEN; l++) {
    offs[l] = o;
    o += count[l];
  }
  {
    int fill[17];
    memcpy(fill, offs, sizeof fill);
    for (int s = 0; s < A; s++)
      if (len[s]) sorted[fill[len[s]]++] = s;
  }
  for (int l = 1; l <= MAXLEN; l++) {
    code = (code + (uint32_t)count[l - 1]) << 1;
    first[l] = (int)code;
  }
  uint64_t total_bits = 0;
  for (int j = 0; j < nseg; j++) total_bits += get_u16(q + 2 * j);
  if (pay != 4 * ((total_bits + 31) / 32)) return ZNO_ERR_CORRUPT;
  uint64_t seg_start = 0;
  for (int j = 0; j < nseg; j++) {
    uint64_t sb = get_u16(q + 2 * j);
    bitr br = {payload, seg_start, seg_start + sb};
    for (uint64_t i = (uint64_t)j * STRIP; i < n;
         i = ((i + 1) % STRIP) ? i + 1 : i + 1 + (uint64_t)(nseg - 1) * STRIP) {
      int c = 0, found = -1;
      for (int l = 1; l <= MAXLEN; l++) {
        unsigned bit;
        if (get_bit(&br, &bit)) return ZNO_ERR_CORRUPT;
        c = (c << 1) | (int)bit;
        if (c >= first[l] && c - first[l] < count[l]) {
          found = sorted[offs[l] + c - first[l]];
          break;
        }
      }
      if (found < 0) return ZNO_ERR_CORRUPT;
      sym[i] = (uint8_t)found;
    }
    if (br.pos != br.end) return ZNO_ERR_CORRUPT; /* segment length must be exact */
    seg_start += sb;
  }
  return (int64_t)(head + align16(pay));
}

int zno_decompress(const void *inv, uint64_t in_bytes, const zno_tableset *ts, void *const *outs,
                   const uint64_t *n_expect, int T_expect) {
  const uint8_t *in = (const uint8_t *)inv;
  int dt, T;
  uint64_t ntot, total, hash;
  uint32_t cb, M;
  int rc = zno_header(in, in_bytes, &dt, &T, &ntot, &cb, &M, &total, &hash);
  if (rc < 0) return rc;
  if (total > in_bytes || T < 1 || (uint64_t)T > in_bytes / 16) return ZNO_ERR_CORRUPT;
  if (64 + 16 * (uint64_t)T + 16 > total) return ZNO_ERR_CORRUPT;
  if (T != T_expect || !outs || !n_expect) return ZNO_ERR_ARG;
  int grouped = in[7] & 1;
  if (grouped && (!ts || ts->K == 0 || ts->hash != hash)) return ZNO_ERR_TABLESET;
  if (!grouped && hash != 0) return ZNO_ERR_CORRUPT;
  uint64_t off_dir = get_u64(in + 40), off_rec = get_u64(in + 48);
  if (off_dir != 64 + 16 * (uint64_t)T) return ZNO_ERR_CORRUPT;
  uint64_t *n = (uint64_t *)calloc((size_t)T, 8), *raw_off = (uint64_t *)calloc((size_t)T, 8);
  if (!n || !raw_off) {
    free(n), free(raw_off);
    return ZNO_ERR_NOMEM;
  }
  uint64_t nsum = 0;
  for (int t = 0; t < T; t++) {
    n[t] = get_u64(in + 64 + 16 * (uint64_t)t);
    nsum += n[t];
  }
  layout lo;
  rc = ZNO_OK;
  for (int t = 0; t < T; t++)
    if (n[t] != n_expect[t] || n[t] > ((uint64_t)1 << 40)) rc = ZNO_ERR_CORRUPT;
  if (rc == ZNO_OK) {
    make_layout(dt, n, T, cb, raw_off, &lo);
    if (nsum != ntot || lo.n_chunks != M || lo.off_records != off_rec || off_rec + 16 > total)
      rc = ZNO_ERR_CORRUPT;
    for (int t = 0; t < T && rc == ZNO_OK; t++)
      if (get_u64(in + 72 + 16 * (uint64_t)t) != raw_off[t]) rc = ZNO_ERR_CORRUPT;
  }
  if (rc == ZNO_OK && get_u64(in + off_dir + 8 * (uint64_t)M) != total - 16) rc = ZNO_ERR_CORRUPT;
  uint64_t ce = chunk_elems(dt, cb);
  uint8_t *sym = (uint8_t *)malloc((size_t)ce * 4);
  if (!sym) rc = ZNO_ERR_NOMEM;
  int nc = ncoded(dt), S = segsyms(dt);
  uint32_t c = 0;
  for (int t = 0; t < T && rc == ZNO_OK; t++) {
    uint8_t *o = (uint8_t *)outs[t];
    for (uint64_t i0 = 0; i0 < n[t] && rc == ZNO_OK; i0 += ce, c++) {
      uint64_t m = n[t] - i0 < ce ? n[t] - i0 : ce;
      uint64_t r0 = get_u64(in + off_dir + 8 * (uint64_t)c), r1 = get_u64(in + off_dir + 8 * (uint64_t)c + 8);
      if (r0 < off_rec || r1 < r0 || r1 > total - 16 || (r0 & 15)) {
        rc = ZNO_ERR_CORRUPT;
        break;
      }
      const uint8_t *sec = in + r0;
      for (int p = 0; p < nc; p++) {
        int64_t sz = decode_stream(sec, in + r1, m, kbits(dt, p), S, ts, grouped && p == 0, p == 0,
                                   sym + (uint64_t)p * m);
        if (sz < 0) {
          rc = (int)sz;
          break;
        }
        sec += sz;
      }
      if (rc == ZNO_OK && sec != in + r1) rc = ZNO_ERR_CORRUPT;
      for (uint64_t i = 0; i < m && rc == ZNO_OK; i++) {
        uint8_t s4[4] = {0, 0, 0, 0};
        uint32_t raw = 0;
        for (int p = 0; p < nc; p++) s4[p] = sym[(uint64_t)p * m + i];
        uint64_t e = i0 + i;
        if (dt == ZNO_BF16) raw = in[raw_off[t] + e];
        if (dt == ZNO_FP8_E4M3) raw = (in[raw_off[t] + e / 8] >> (e % 8)) & 1;
        if (dt == ZNO_FP4X2_E2M1) raw = (in[raw_off[t] + e / 4] >> (2 * (e % 4))) & 3;
        store_elem(dt, o, e, merge_one(dt, s4, raw));
      }
    }
  }
  free(sym), free(n), free(raw_off);
  return rc;
}
