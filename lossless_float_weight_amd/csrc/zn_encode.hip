// zn_encode.hip -- the compression pass for gfx950.
//
// Three launches, each chunk-parallel or tiny:
//   k_analyze (one workgroup per chunk; 4 wave64s for BF16, 8 otherwise)
//   1. reads the chunk once with 16-byte loads, splits every element into its
//      coded fields and its always-raw bits (THEORY-599 on ZipNN, per-field
//      compressibility, ZipNN Table II), stores the raw bits straight to their
//      final place, and counts each coded field in LDS histograms privatised
//      per lane column (the exponent histogram is very skewed: a handful of
//      bins take most hits, so lanes must not share counters);
//   2. per coded stream chooses constant / shared group code / own optimal
//      code / raw by exact section size; the own code is built in LDS by
//      package-merge (THEORY-599, order-0 only; "NeuralZip: Reusable Setup
//      for Fast Lossless Compression", Abstract, for group codes).  The
//      choice, the code words and the record size go to a per-chunk plan.
//   k_finish (one workgroup) scans the record sizes into the directory and
//   writes the header and the alignment gaps.
//   k_pack (one workgroup of 4 wave64s per chunk) writes the chunk's record
//   at its directory offset: stream heads, then each coded payload in tiles
//   of whole segments (one or two per wave) -- a wave scan of bit counts, code
//   words ORed into an LDS tile, whole words stored coalesced -- and the raw
//   streams, from those tiles where their words allow (through rings per
//   strip row that store whole 128-byte lines), else in a pass of their own.
// No chunk ever waits for another, and no record is copied after packing.
#include <type_traits>

#include "zn_internal.h"

namespace zn {

// threads per chunk in k_analyze: BF16 chunks use 256 so that every chunk of
// a large workload is resident at once (7 workgroups of under 20 KB LDS per
// CU); k_pack always uses 256.
constexpr int enc_nt(int dt) { return dt == BF16 ? 256 : 512; }
constexpr int PACK_NT = 256, PACK_NW = PACK_NT / 64;

// Per-chunk plan, written by k_analyze and read by k_pack:
//   u64 bits[4] (payload bits per coded stream), u32 sec_off[4] (offset of
//   each stream's section in the record), u8 mode[4], u8 aux[4], pad to 64,
//   then u32 enc[ncoded][256] (bit-reversed code | length << 16) for the
//   streams coded with a Huffman or group code, or the normalised counts of
//   a tANS-coded stream; then (tANS) the u16 bit length of each segment of
//   the first stream.
__host__ __device__ constexpr uint64_t plan_fixed(int dt) { return 64 + 1024ull * ncoded(dt); }

template <int DT, int P>
__device__ __forceinline__ uint32_t field(uint32_t w) {
  if constexpr (DT == BF16) return (w >> 7) & 0xFF;
  if constexpr (DT == FP32) {
    if constexpr (P == 0) return (w >> 23) & 0xFF;
    if constexpr (P == 1) return ((w >> 24) & 0x80) | ((w >> 16) & 0x7F);
    if constexpr (P == 2) return (w >> 8) & 0xFF;
    return w & 0xFF;
  }
  if constexpr (DT == FP4X2) {   // the byte's two exponents, then its two mantissas
    if constexpr (P == 0) return ((w >> 1) & 3) | ((w >> 3) & 0xC);
    return (w & 1) | ((w >> 3) & 2);
  }
  if constexpr (P == 0) return (w >> 3) & 0xF;
  return w & 7;
}

template <int DT>
__device__ __forceinline__ uint32_t field_rt(uint32_t w, int p) {
  if constexpr (DT == BF16) return field<DT, 0>(w);
  if constexpr (DT == FP32) {
    switch (p) {
      case 0: return field<DT, 0>(w);
      case 1: return field<DT, 1>(w);
      case 2: return field<DT, 2>(w);
      default: return field<DT, 3>(w);
    }
  }
  return p == 0 ? field<DT, 0>(w) : field<DT, 1>(w);
}

// The first stream's field of each of a word's four 1-byte elements, in
// that element's byte.
template <int DT>
__device__ __forceinline__ uint32_t field0_4(uint32_t x) {
  static_assert(DT == FP8 || DT == FP4X2, "1-byte elements");
  if constexpr (DT == FP4X2) return ((x >> 1) & 0x03030303u) | ((x >> 3) & 0x0C0C0C0Cu);
  return (x >> 3) & 0x0F0F0F0Fu;
}

// element i of a 16-byte vector
template <int DT>
__device__ __forceinline__ uint32_t vec_elem(const uint4 &q, int i) {
  constexpr int ES = esize(DT);
  const int byte = i * ES;
  const uint32_t x = (byte >> 2) == 0 ? q.x : (byte >> 2) == 1 ? q.y : (byte >> 2) == 2 ? q.z : q.w;
  if constexpr (ES == 4) return x;
  if constexpr (ES == 2) return (x >> ((byte & 2) * 8)) & 0xFFFF;
  return (x >> ((byte & 3) * 8)) & 0xFF;
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem(const uint8_t *p) {
  if constexpr (DT == BF16) return ldg1(p) | (ldg1(p + 1) << 8);
  if constexpr (DT == FP32) return ldg1(p) | (ldg1(p + 1) << 8) | (ldg1(p + 2) << 16) | (ldg1(p + 3) << 24);
  return ldg1(p);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Segments per wave in one pack tile: 16 symbols per lane per tile (more
// per tile holds fewer workgroups per CU than the chunks need); FP32, whose
// tiles also carry three raw streams, takes 8 (80 VGPRs: 6 workgroups per CU
// instead of 4 at 16).
constexpr int pack_g(int dt) { return dt == FP32 ? 2 : segsyms(dt) / 64 >= 16 ? 1 : 16 / (segsyms(dt) / 64); }

// The mantissa fields of a word's four 1-byte elements, element 0 in the low
// bits (FP8: 3 bits each; FP4 pairs: the byte's two mantissa bits, low nibble's first).
template <int DT>
__device__ __forceinline__ uint32_t mant4(uint32_t x) {
  if constexpr (DT == FP8) {
    const uint32_t m = x & 0x07070707u, t = m | (m >> 5);
    return (t & 0x3Fu) | ((t >> 10) & 0xFC0u);
  } else {
    const uint32_t m = (x & 0x01010101u) | ((x >> 3) & 0x02020202u), t = m | (m >> 6);
    return (t & 0xFu) | ((t >> 12) & 0xF0u);
  }
}

// LDS of a tANS encoder: table construction, then the state of each
// (symbol, rank) and each symbol's step constants.
template <int NT>
struct TansEnc {
  TansBuild<NT> tb;
  uint16_t est[kTansStates];
  uint32_t esym[256];
};

// Encodes segment j of the first coded stream of a chunk of n elements at
// src with tANS, backwards: its strips j + r*nseg (32 elements each) from the
// last to the first, each from its last element.  emit(v, nb) receives each
// symbol's bits in that order.  Returns the final state minus 2^11.
// Per strip: the strip's 32 symbols are taken out of its loaded vectors
// (held in registers from then on), then hook() runs (the packer stores
// what the previous strip completed), then the next strip's vectors are
// loaded, then the symbols are encoded.  No global store comes between a
// load and the wait for it: the one counter of outstanding vector memory
// operations would otherwise make that wait drain the stores too.
template <int DT, class Emit, class Hook>
__device__ __forceinline__ uint32_t tans_encode_segment(const uint8_t *src, uint32_t n, bool aligned, int nseg,
                                                        int j, const uint32_t *esym, const uint16_t *est,
                                                        Emit &&emit, Hook &&hook) {
  constexpr int ES = esize(DT), VE = 16 / ES, NQ = 32 * ES / 16;
  const uint32_t nstrips = (n + 31) / 32;
  uint32_t X = kTansStates;
  auto load = [&](uint32_t q, u32x4 (&v)[NQ]) {
    const uint32_t eb = q * 32;
    if (aligned && eb + 32 <= n) {
#pragma unroll
      for (int i = 0; i < NQ; i++) v[i] = ldg16(src + uint64_t(eb) * ES + 16 * i);
    } else {
#pragma unroll
      for (int i = 0; i < NQ; i++) v[i] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 32; e++) {
        const uint32_t w = eb + e < n ? load_elem<DT>(src + uint64_t(eb + e) * ES) : 0u;
        const int b = e * ES;
        v[b >> 4][(b >> 2) & 3] |= w << ((b & 3) * 8);
      }
    }
  };
  if (uint32_t(j) >= nstrips) return 0;   // not reached: a stream has no more segments than strips
  const uint32_t ql = uint32_t(j) + (nstrips - 1 - uint32_t(j)) / uint32_t(nseg) * uint32_t(nseg);
  u32x4 raw[NQ];
  load(ql, raw);
  for (int64_t q = ql; q >= j; q -= nseg) {
    // the strip's symbols, four to a register (every field is at most 8 bits)
    uint32_t sy[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int e = 4 * k + i;
        const u32x4 c4 = raw[e / VE];
        x |= field<DT, 0>(vec_elem<DT>(make_uint4(c4[0], c4[1], c4[2], c4[3]), e % VE)) << (8 * i);
      }
      sy[k] = x;
      asm volatile("" : "+v"(sy[k]));   // taken here, before the hook's stores and the next loads
    }
    hook();
    if (q - nseg >= j) load(uint32_t(q - nseg), raw);
    const uint32_t eb = uint32_t(q) * 32;
    const uint32_t lim = n - eb < 32 ? n - eb : 32u;
    // each symbol's step constants are read one step ahead, so that a step
    // waits for one LDS read (the next state), not two
    auto symb = [&](int e) { return (sy[e >> 2] >> (8 * (e & 3))) & 0xFFu; };
    uint32_t info = esym[symb(31)];
#pragma unroll
    for (int e = 31; e >= 0; e--) {
      const uint32_t next = e > 0 ? esym[symb(e > 0 ? e - 1 : 0)] : 0u;
      if (uint32_t(e) < lim) {
        uint32_t v;
        const uint32_t nb = tans_enc_step(X, info, est, v);
        emit(v, nb);
      }
      info = next;
    }
  }
  return X - kTansStates;
}

// Writes one segment's bits [b0, b1) of a payload backwards, as tANS emits
// them: acc holds words T-1 (low half) and T (high half), and word T is done
// once the bits reach below word T-1.  Done words go to the lane's 16-word
// ring in LDS (word w at w mod 16); store() writes the 4-word blocks whose
// words are all done, a whole aligned block as one 16-byte store: every lane
// of a wave writes a segment of its own, so word stores would leave lines
// partly written in the L2.  The words the segment shares with its
// neighbours (its first and last, when not word-aligned) are ORed
// atomically at the end into words cleared beforehand.  A strip adds at
// most 11 words (32 symbols of at most 11 bits) to at most 3 not yet stored,
// so the ring never wraps onto a word not yet stored.
struct RingWriter {
  uint32_t *pw, *lb;
  int32_t b0, b1, cur, T, fw, lw, ofw, olw, wl, pend;
  uint32_t topw, botw;
  uint64_t acc;
  __device__ RingWriter(uint32_t *p, uint32_t *ring, int32_t lo, int32_t hi)
      : pw(p), lb(ring), b0(lo), b1(hi), cur(hi), T((hi - 1) >> 5), fw(lo >> 5), lw((hi - 1) >> 5),
        topw(0), botw(0), acc(0) {
    ofw = fw + ((lo & 31) != 0);   // the words this segment alone holds: [ofw, olw]
    olw = lw - ((hi & 31) != 0);
    wl = olw + 1;                  // lowest word done so far
    pend = olw >> 2;               // highest block not yet stored
  }
  __device__ __forceinline__ void word(int32_t w, uint32_t x) {
    if (w == lw && (b1 & 31)) topw = x;
    else if (w == fw && (b0 & 31)) botw = x;
    else {
      lb[w & 15] = x;
      wl = w;
    }
  }
  __device__ __forceinline__ void block(int32_t B) {
    const int32_t w0 = 4 * B;
    if (w0 >= ofw && w0 + 3 <= olw) {
      stg16(pw + w0, *reinterpret_cast<const u32x4 *>(lb + (w0 & 15)));
    } else {
#pragma unroll
      for (int k = 0; k < 4; k++)
        if (w0 + k >= ofw && w0 + k <= olw) stg4(pw + w0 + k, lb[(w0 + k) & 15]);
    }
  }
  // the blocks whose owned words are all done
  __device__ __forceinline__ void store() {
    const int32_t lowb = (wl + 3) >> 2;
    for (; pend >= lowb; pend--) block(pend);
  }
  __device__ __forceinline__ void put(uint32_t v, uint32_t nb) {
    const int32_t pos = cur - int32_t(nb);
    if (pos < 32 * (T - 1)) {
      word(T, uint32_t(acc >> 32));
      acc <<= 32;
      T--;
    }
    acc |= uint64_t(v) << ((pos - 32 * (T - 1)) & 63);   // nb = 0 ORs nothing
    cur = pos;
  }
  // after the final state: the last words, every block left, the shared words
  __device__ __forceinline__ void finish() {
    word(T, uint32_t(acc >> 32));
    if (fw == T - 1) word(T - 1, uint32_t(acc));
    for (; pend >= (ofw >> 2); pend--) block(pend);
    if (b1 & 31)
      __hip_atomic_fetch_or((ZN_GLOBAL uint32_t *)(pw + lw), topw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((b0 & 31) && !(fw == lw && (b1 & 31)))
      __hip_atomic_fetch_or((ZN_GLOBAL uint32_t *)(pw + fw), botw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// LDS of the tANS packing: the encoder tables and each lane's word ring.
struct TansPack {
  TansEnc<PACK_NT> e;
  alignas(16) uint32_t ring[PACK_NT][16];
};

template <int DT, bool TC = false>
struct PackShared {
  static constexpr int NC = ncoded(DT);
  static constexpr int G = pack_g(DT);
  // words of one tile at the longest codes, plus slack for the group ORs
  static constexpr int STAGE = (PACK_NW * G * segsyms(DT) * kMaxLen + 31) / 32 + 4;
  uint32_t enc[NC][256];         // tANS: the first stream's normalised counts
  union {
    uint32_t stage[2][STAGE];    // alternate tiles use alternate buffers
    // a tANS stream's tables and write buffers (no tiles meanwhile); only
    // the kernels that pack tANS hold them
    std::conditional_t<TC, TansPack, uint32_t> tans;
  } su;
  uint32_t wtot[2][PACK_NW];
  // BF16 chunks of a group that packs exponent pairs: the pair tokens' codes
  // and F's ranks
  static constexpr int PA = DT == BF16 ? 256 : 1;
  uint32_t penc[PA];
  uint8_t prk[PA];
  // 1-byte elements: the first stream's codes joined for two consecutive
  // symbols x, y at entry x + 16 y (rows 0..15), the single code of x at
  // 256 + x and nothing at 272..287 (for a run's elements past the chunk's
  // end); the code word in bits 0..21, its bit count in bits 27..31
  static constexpr int P2 = DT == FP8 || DT == FP4X2 ? 288 : 1;
  uint32_t enc2[P2];
  // 1-byte elements: the raw mantissa stream's words (32 strips per
  // segment, kbits words per strip), written from the coded stream's tiles
  // into a ring per strip row.  After each group of RT tiles a row stores
  // the whole 128-byte lines it now holds and keeps the rest (under a line)
  // for the next group, so no store leaves a line part-written (the per-tile
  // runs are 48 bytes for FP8 and 32 for FP4 pairs, parts of lines that the
  // L2 wrote back before the next tiles filled them).  The ring holds a
  // group and the rest before it (RW >= GW + 28); it is a whole number of
  // strips and of 16-byte vectors, and small enough to keep six workgroups
  // per CU.  A chunk whose first stream is tANS-coded never takes this path,
  // so the tANS kernels hold no ring.
  static constexpr bool RSTAGE = (DT == FP8 || DT == FP4X2) && !TC;
  static constexpr int RT = 4;
  static constexpr int GW = RT * PACK_NW * G * kbits(DT, 1);      // a group's words per row
  static constexpr int RW = DT == FP8 ? 84 : 64;                  // ring words per row
  static_assert(!RSTAGE || (RW >= GW + 28 && RW % kbits(DT, 1) == 0 && RW % 4 == 0), "ring size");
  uint32_t rawt[RSTAGE ? 32 * RW : 1];
  // FP32: the same for the raw fraction-byte streams written from the first
  // coded stream's tiles (up to three streams, 8 strip rows each, 64 words
  // of a row per tile, stored after every tile), in chunks of whole segments
  static constexpr bool FRING = DT == FP32 && !TC;
  static constexpr int FW = 128;                                  // ring words per row (a power of two)
  uint32_t fring[FRING ? 3 * 8 * FW : 1];
  unsigned long long bits[NC], sec_off[NC];
  int mode[NC], aux[NC];
};

template <int DT>
struct EncShared {
  static constexpr int NC = ncoded(DT);
  static constexpr int S = segsyms(DT);
  static constexpr int NT = enc_nt(DT);
  static constexpr int NW = NT / 64;                              // waves = segments per pack tile
  static constexpr int COLS = DT == FP32 ? 16 : 32;
  // 1-byte elements count whole bytes (one bin of 256 per element) and take
  // their two fields' histograms from that; the others count each field
  static constexpr bool BYTEHIST = DT == FP8 || DT == FP4X2;
  static constexpr int APRIV = BYTEHIST ? 256 : 256 * NC;   // total bins
  // BF16 counts two bins per word (a column sees at most 1/32 of a chunk,
  // 16384 values at the largest chunk size, so 16 bits cannot overflow), to
  // keep every chunk of a block resident at once; the others count one bin
  // per word (for 1-byte elements the bin's address is then two instructions
  // from the byte, and the histogram 32 KB)
  static constexpr bool PACK16 = DT == BF16;
  static constexpr int PRIVW = PACK16 ? APRIV * COLS / 2 : APRIV * COLS;
  uint32_t hist[NC][256];
  uint32_t enc[NC][256];   // tANS: the first stream's normalised counts
  uint8_t len[NC][256];
  unsigned long long bits[NC];
  unsigned long long sec_off[NC + 1];
  int mode[NC], aux[NC];
  unsigned long long rsum[NW];
  int icnt[NW];
  int cnt[4][kMaxLen + 1];
  int need_block, need_tans, tans_d;
  union {
    uint32_t priv[PRIVW];
    struct {
      PMShared pm;
      uint64_t hw[256];
    } cb;
    WaveCB wcb;
    TansEnc<NT> tans;
  } u;
};

template <int DT>
__device__ __forceinline__ int priv_base(int p) {
  return p * 256;
}

// Block-wide sum of one value per thread (u64).
template <int DT>
__device__ unsigned long long block_sum(EncShared<DT> &sh, unsigned long long v) {
  const int tid = threadIdx.x;
  v = wave_sum_u64(v);
  __syncthreads();
  if ((tid & 63) == 0) sh.rsum[tid >> 6] = v;
  __syncthreads();
  unsigned long long t = 0;
  for (int w = 0; w < EncShared<DT>::NW; w++) t += sh.rsum[w];
  return t;
}
template <int DT>
__device__ int block_count(EncShared<DT> &sh, bool pred) {
  const int tid = threadIdx.x;
  const int c = __popcll(__ballot(pred));
  __syncthreads();
  if ((tid & 63) == 0) sh.icnt[tid >> 6] = c;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < EncShared<DT>::NW; w++) t += sh.icnt[w];
  return t;
}

// one histogram count of field value b of stream p, in column col
template <int DT>
__device__ __forceinline__ void count(EncShared<DT> &sh, int p, uint32_t b, int col) {
  constexpr int COLS = EncShared<DT>::COLS;
  const uint32_t bin = priv_base<DT>(p) + b;
  if constexpr (EncShared<DT>::PACK16)
    atomicAdd(&sh.u.priv[(bin >> 1) * COLS + col], 1u << (16 * (bin & 1)));
  else
    atomicAdd(&sh.u.priv[bin * COLS + col], 1u);
}

// Steps 1 and 2 for chunk c: raw planes stored, histograms, and per coded
// stream the mode, code and section offset in sh.  Returns the record size.
// TC: the exponent stream takes the tANS coder (chunks with their own
// counts; no group tables), its segments' bit lengths going to segbits.
template <int DT, bool TC>
__device__ __forceinline__ uint64_t analyze_chunk(const EncArgs &a, EncShared<DT> &sh, uint32_t c,
                                                  uint8_t *segbits) {
  constexpr int NC = ncoded(DT), ES = esize(DT), S = segsyms(DT);
  constexpr int VE = 16 / ES;          // elements per 16-byte vector
  constexpr int COLS = EncShared<DT>::COLS;
  constexpr int ENC_NT = EncShared<DT>::NT;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;

  const int t = find_tensor(a.L, c);
  const uint64_t e0 = uint64_t(c - a.L.t_chunk0[t]) * a.L.chunk_elems;
  const uint64_t rem = a.L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < a.L.chunk_elems ? rem : a.L.chunk_elems);
  const uint8_t *src = a.in_ptrs[t] + e0 * ES;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const uint32_t nvec = aligned ? n / VE : 0;
  uint8_t *rawp = a.out + a.L.t_raw[t];

  // ------- 0. BF16 with a group code that packs exponent pairs: no histogram
  // The setup chose the chunk's code, which codes the aligned pairs of values
  // of the group's F that have a pair code as one token ("NeuralZip",
  // Abstract: recurring tuples as packed exponents).  What the mode choice
  // needs is the coded size under it, whether every exponent present has a
  // code word, and whether only one exponent value occurs (constant).  All
  // three come from one 64-bit LDS table entry per exponent value (the token
  // code's single lengths), a pair's entry taking its pair code's length
  // when it has one, summed per thread: the code length (bits 0-15), 1 if it
  // has no code word (bits 16-31), 1 if it equals the chunk's first exponent
  // (bits 32-47); a thread sums at most 2048 entries of at most 11, so no
  // field overflows.  A chunk with an exponent its group lacks (an escape) is
  // counted below like any other.  Chunks of the other groups take the
  // histogram below: with it an escape needs no second read of the chunk, and
  // on the perturbed full model (about one chunk in six escapes) the
  // analysis takes 6.2 ms with it against 6.6 ms with this path.
  if constexpr (DT == BF16) {
    const int g = a.group_map ? int(ldg1(a.group_map + c)) : 0;
    if (a.group_map && a.group_packed && ldg1(a.group_packed + g)) {
      const uint32_t ef = (load_elem<DT>(src) >> 7) & 0xFF;   // the chunk's first exponent
      unsigned long long *tbl = reinterpret_cast<unsigned long long *>(sh.u.priv);
      uint8_t *rk = reinterpret_cast<uint8_t *>(sh.u.priv + 512);        // F's ranks
      uint8_t *plen = reinterpret_cast<uint8_t *>(sh.u.priv + 576);      // pair code lengths
      if (tid < 256) {
        const uint32_t l = ldg1(a.group_len + g * 256 + tid);
        tbl[tid] = l | (uint64_t(l == 0) << 16) | (uint64_t(uint32_t(tid) == ef) << 32);
        rk[tid] = uint8_t(ldg1(a.group_rank + g * 256 + tid));
        plen[tid] = uint8_t(ldg4(a.group_penc + g * 256 + tid) >> 16);
      }
      __syncthreads();
      // one aligned pair's entry: the pair code's length (bits 0-15) with
      // the two values' "equals the first" counts, or the two singles
      auto pair_cost = [&](uint32_t x, uint32_t y) -> unsigned long long {
        const unsigned long long sxy = tbl[x] + tbl[y];
        const uint32_t rx = rk[x], ry = rk[y];
        const uint32_t pl = (rx | ry) < 16 ? plen[16 * rx + ry] : 0u;
        return pl ? (sxy & ~0xFFFFFFFFull) | pl : sxy;
      };
      unsigned long long acc = 0;
      constexpr int B0 = 4;  // 16-byte loads in flight per thread
      for (uint32_t v0 = tid; v0 < nvec; v0 += B0 * ENC_NT) {
        u32x4 qs[B0];
#pragma unroll
        for (int b = 0; b < B0; b++) {
          const uint32_t v = v0 + b * ENC_NT;
          if (v < nvec) qs[b] = ldg16(src + 16ull * v);
        }
#pragma unroll
        for (int b = 0; b < B0; b++) {
          const uint32_t v = v0 + b * ENC_NT;
          if (v >= nvec) break;
          const uint4 q = make_uint4(qs[b][0], qs[b][1], qs[b][2], qs[b][3]);
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int j = 0; j < 4; j++)   // a vector holds 4 aligned pairs
            acc += pair_cost((vec_elem<DT>(q, 2 * j) >> 7) & 0xFF, (vec_elem<DT>(q, 2 * j + 1) >> 7) & 0xFF);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint32_t w0 = vec_elem<DT>(q, i), w1 = vec_elem<DT>(q, i + 4);
            lo |= (((w0 >> 8) & 0x80) | (w0 & 0x7F)) << (8 * i);
            hi |= (((w1 >> 8) & 0x80) | (w1 & 0x7F)) << (8 * i);
          }
          stg8(rawp + e0 + uint64_t(v) * 8, u32x2{lo, hi});
        }
      }
      // ragged tail or unaligned input: pairs from even positions
      for (uint32_t i = nvec * VE + 2 * tid; i < n; i += 2 * ENC_NT) {
        const uint32_t w = load_elem<DT>(src + uint64_t(i) * ES);
        stg1(rawp + e0 + i, ((w >> 8) & 0x80) | (w & 0x7F));
        if (i + 1 < n) {
          const uint32_t w1 = load_elem<DT>(src + uint64_t(i + 1) * ES);
          stg1(rawp + e0 + i + 1, ((w1 >> 8) & 0x80) | (w1 & 0x7F));
          acc += pair_cost((w >> 7) & 0xFF, (w1 >> 7) & 0xFF);
        } else {
          acc += tbl[(w >> 7) & 0xFF];   // a lone last value
        }
      }
      const unsigned long long bits = block_sum<DT>(sh, acc & 0xFFFFu);
      const unsigned long long nmiss = block_sum<DT>(sh, (acc >> 16) & 0xFFFFu);
      const unsigned long long nfirst = block_sum<DT>(sh, (acc >> 32) & 0xFFFFu);
      const int nseg = int((n + S - 1) / S);
      const unsigned long long raw = section_bytes(RAW, 8, n, nseg, 0);
      if (nfirst == n || nmiss == 0) {
        int mode = RAW, aux = 0;
        if (nfirst == n) {
          mode = CONST;
          aux = int(ef);
        } else if (section_bytes(GROUP, 8, n, nseg, bits) < raw) {
          mode = GROUP;
          aux = g;
        }
        if (tid < 256)
          sh.enc[0][tid] = mode == GROUP ? ldg4(a.group_enc + g * 256 + tid)
                                         : uint32_t(tid) | (8u << 16);
        if (tid == 0) {
          sh.mode[0] = mode;
          sh.aux[0] = aux;
          sh.bits[0] = mode == GROUP ? bits : mode == RAW ? uint64_t(n) * 8 : 0;
          sh.sec_off[0] = 0;
        }
        __syncthreads();
        return section_bytes(mode, 8, n, nseg, mode == GROUP ? bits : 0);
      }
      __syncthreads();   // an escape: the histogram below decides
    }
  }

  // ------------------------------------------- 1. split, raw planes, counts
  for (int i = tid; i < EncShared<DT>::PRIVW; i += ENC_NT) sh.u.priv[i] = 0;
  if constexpr (EncShared<DT>::BYTEHIST) {   // the field histograms are summed into
    for (int i = tid; i < NC * 256; i += ENC_NT) sh.hist[i >> 8][i & 255] = 0;
  }
  __syncthreads();
  const int col = ln & (COLS - 1);
  constexpr int B1 = 4;  // 16-byte loads in flight per thread
  for (uint32_t v0 = tid; v0 < nvec; v0 += B1 * ENC_NT) {
    u32x4 qs[B1];
#pragma unroll
    for (int b = 0; b < B1; b++) {
      const uint32_t v = v0 + b * ENC_NT;
      if (v < nvec) qs[b] = ldg16(src + 16ull * v);
    }
#pragma unroll
    for (int b = 0; b < B1; b++) {
      const uint32_t v = v0 + b * ENC_NT;
      if (v >= nvec) break;
      const uint4 q = make_uint4(qs[b][0], qs[b][1], qs[b][2], qs[b][3]);
#pragma unroll
      for (int i = 0; i < VE; i++) {
        const uint32_t w = vec_elem<DT>(q, i);
        if constexpr (EncShared<DT>::BYTEHIST) {
          count<DT>(sh, 0, w, col);
        } else {
#pragma unroll
          for (int p = 0; p < NC; p++) count<DT>(sh, p, field_rt<DT>(w, p), col);
        }
      }
      if constexpr (DT == BF16) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint32_t w0 = vec_elem<DT>(q, i), w1 = vec_elem<DT>(q, i + 4);
          lo |= (((w0 >> 8) & 0x80) | (w0 & 0x7F)) << (8 * i);
          hi |= (((w1 >> 8) & 0x80) | (w1 & 0x7F)) << (8 * i);
        }
        stg8(rawp + e0 + uint64_t(v) * 8, u32x2{lo, hi});
      } else if constexpr (DT == FP8) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) m |= ((vec_elem<DT>(q, i) >> 7) & 1) << i;
        stg2(rawp + e0 / 8 + uint64_t(v) * 2, m);
      } else if constexpr (DT == FP4X2) {   // the two sign bits of each byte
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const uint32_t w = vec_elem<DT>(q, i);
          m |= (((w >> 3) & 1) | ((w >> 6) & 2)) << (2 * i);
        }
        stg4(rawp + e0 / 4 + uint64_t(v) * 4, m);
      }
    }
  }
  for (uint32_t i = nvec * VE + tid; i < n; i += ENC_NT) {  // ragged tail or unaligned input
    const uint32_t w = load_elem<DT>(src + uint64_t(i) * ES);
    if constexpr (EncShared<DT>::BYTEHIST) {
      count<DT>(sh, 0, w, col);
    } else {
#pragma unroll
      for (int p = 0; p < NC; p++) count<DT>(sh, p, field_rt<DT>(w, p), col);
    }
    if constexpr (DT == BF16) stg1(rawp + e0 + i, ((w >> 8) & 0x80) | (w & 0x7F));
  }
  if constexpr (DT == FP8) {  // sign bits of the tail, whole bytes by one thread
    if (tid == 0 && nvec * VE < n) {
      for (uint32_t b = nvec * VE / 8; b < (n + 7) / 8; b++) {
        uint32_t m = 0;
        for (uint32_t i = b * 8; i < b * 8 + 8 && i < n; i++)
          m |= ((uint32_t(src[i]) >> 7) & 1) << (i - b * 8);
        rawp[e0 / 8 + b] = uint8_t(m);
      }
    }
  }
  if constexpr (DT == FP4X2) {  // sign pairs of the tail, whole bytes by one thread
    if (tid == 0 && nvec * VE < n) {
      for (uint32_t b = nvec * VE / 4; b < (n + 3) / 4; b++) {
        uint32_t m = 0;
        for (uint32_t i = b * 4; i < b * 4 + 4 && i < n; i++) {
          const uint32_t w = src[i];
          m |= (((w >> 3) & 1) | ((w >> 6) & 2)) << (2 * (i - b * 4));
        }
        rawp[e0 / 4 + b] = uint8_t(m);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < EncShared<DT>::APRIV; i += ENC_NT) {
    uint32_t s = 0;
    if constexpr (EncShared<DT>::PACK16) {
      const int sh16 = 16 * (i & 1);
      for (int j = 0; j < COLS; j++)
        s += (sh.u.priv[(i >> 1) * COLS + ((j + (i >> 1)) & (COLS - 1))] >> sh16) & 0xFFFF;
    } else {
      for (int j = 0; j < COLS; j++) s += sh.u.priv[i * COLS + ((j + i) & (COLS - 1))];
    }
    if constexpr (EncShared<DT>::BYTEHIST) {
      // byte i's count goes to its value of each field
      atomicAdd(&sh.hist[0][field_rt<DT>(uint32_t(i), 0)], s);
      atomicAdd(&sh.hist[1][field_rt<DT>(uint32_t(i), 1)], s);
    } else {
      sh.hist[i >> 8][i & 255] = s;
    }
  }
  __syncthreads();

  // --------------------------------------------- 2. mode and code per stream
  const int nseg = int((n + S - 1) / S);
  unsigned long long rec = 0;
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k;
    const unsigned long long raw = section_bytes(RAW, k, n, nseg, 0);
    // wave 0 decides the mode and builds the code; the workgroup helps only
    // when more than 64 symbols are present
    if (wv == 0) {
      uint32_t hq[4];
      uint64_t mq[4];
      int d = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int s2 = ln + 64 * q;
        hq[q] = s2 < A ? sh.hist[p][s2] : 0u;
        mq[q] = __ballot(hq[q] != 0);
        d += __popcll(mq[q]);
      }
      int mode = RAW, aux = 0, need_block = 0, need_tans = 0;
      uint64_t bits = 0;
      if (d == 1) {
        mode = CONST;
#pragma unroll
        for (int q = 3; q >= 0; q--)
          if (mq[q]) aux = 64 * q + __ffsll((long long)mq[q]) - 1;
      } else if (TC && p == 0) {
        // tANS: the counts here; the size needs every segment encoded (below)
        const int dd = wave_tans_normalize(sh.hist[0], A, n, sh.enc[0]);
        if (ln == 0) sh.tans_d = dd;
        need_tans = 1;
      } else {
        bool escape = true;
        if (p == 0 && a.group_map) {
          const int g = ldg1(a.group_map + c);
          uint32_t gl[4];
          bool miss = false;
          uint64_t part = 0;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int s2 = ln + 64 * q;
            gl[q] = s2 < A ? ldg1(a.group_len + g * 256 + s2) : 0u;
            miss |= hq[q] && !gl[q];
            part += uint64_t(hq[q]) * gl[q];
          }
          if (!__ballot(miss)) {
            escape = false;
            bits = wave_sum64(part);
            if (section_bytes(GROUP, k, n, nseg, bits) < raw) {
              mode = GROUP;
              aux = g;
#pragma unroll
              for (int q = 0; q < 4; q++) {
                const int s2 = ln + 64 * q;
                if (s2 < A) {
                  sh.len[p][s2] = uint8_t(gl[q]);
                  sh.enc[p][s2] = ldg4(a.group_enc + g * 256 + s2);
                }
              }
            }
          }
        }
        // Any prefix code spends at least n*H bits (Shannon's bound from the
        // Kraft inequality), so when even that cannot beat the raw section the
        // optimal code need not be built: the choice is RAW either way.  The
        // bound is taken 64 bits and a relative 1e-9 below the double-precision
        // sum, far more than its rounding error.
        bool raw_sure = false;
        if (escape) {
          double hb = 0.0;
#pragma unroll
          for (int q = 0; q < 4; q++)
            if (hq[q]) hb += double(hq[q]) * log2(double(n) / double(hq[q]));
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) hb += __shfl_xor(hb, o, 64);
          const double lb = hb * (1.0 - 1e-9) - 64.0;
          raw_sure = lb > 0.0 && section_bytes(HUFF, k, n, nseg, uint64_t(lb)) >= raw;
        }
        if (escape && !raw_sure) {
          if (wave_pm_lengths<uint32_t>(sh.hist[p], A, false, sh.len[p], sh.u.wcb) < 0) {
            need_block = 1;
          } else {
            uint64_t part = 0;
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const int s2 = ln + 64 * q;
              if (s2 < A) part += uint64_t(hq[q]) * sh.len[p][s2];
            }
            bits = wave_sum64(part);
            if (section_bytes(HUFF, k, n, nseg, bits) < raw) {
              mode = HUFF;
              wave_canon(sh.len[p], A, sh.enc[p]);
            }
          }
        }
      }
      if (ln == 0) {
        sh.mode[p] = mode;
        sh.aux[p] = aux;
        sh.bits[p] = bits;
        sh.need_block = need_block;
        sh.need_tans = need_tans;
      }
    }
    __syncthreads();
    if constexpr (TC) {
      if (sh.need_tans) {
        // one thread per segment encodes it backwards to count its bits
        auto &T = sh.u.tans;
        tans_tables<ENC_NT>(sh.enc[0], A, T.tb, nullptr, T.est, T.esym);
        unsigned long long acc = 0;
        for (int j = tid; j < nseg; j += ENC_NT) {
          uint32_t nbits = kTansLog;   // the final state, then the symbols' bits
          tans_encode_segment<DT>(src, n, aligned, nseg, j, T.esym, T.est,
                                  [&](uint32_t, uint32_t nb) { nbits += nb; }, [] {});
          stg2(segbits + 2ull * j, nbits);
          acc += nbits;
        }
        const unsigned long long bits = block_sum<DT>(sh, acc);
        if (tid == 0) {
          sh.mode[p] = section_bytes(TANS, k, n, nseg, bits, sh.tans_d) < raw ? TANS : RAW;
          sh.bits[p] = bits;
        }
        __syncthreads();
      }
    }
    if (sh.need_block) {
      const uint32_t h = tid < A ? sh.hist[p][tid] : 0;
      if (tid < A) sh.u.cb.hw[tid] = h;
      __syncthreads();
      pm_lengths<ENC_NT>(sh.u.cb.pm, sh.u.cb.hw, A, false, sh.len[p]);
      const uint8_t l = tid < A ? sh.len[p][tid] : 0;
      const unsigned long long bits = block_sum<DT>(sh, (unsigned long long)h * l);
      const bool huff = section_bytes(HUFF, k, n, nseg, bits) < raw;
      if (huff) canon_encode_table(sh.len[p], A, sh.enc[p], sh.cnt);
      if (tid == 0) {
        sh.mode[p] = huff ? HUFF : RAW;
        sh.bits[p] = bits;
      }
      __syncthreads();
    }
    const int mode = sh.mode[p];
    if (mode == RAW && tid < A) sh.enc[p][tid] = uint32_t(tid) | (uint32_t(k) << 16);
    if (tid == 0) {
      if (mode == RAW) sh.bits[p] = uint64_t(n) * k;
      sh.sec_off[p] = rec;
    }
    rec += section_bytes(mode, k, n, nseg, mode == RAW ? 0 : sh.bits[p], mode == TANS ? sh.tans_d : 0);
    __syncthreads();
  }
  return rec;
}

template <int DT, bool TC>
// BF16: at most 7 waves' worth of registers per SIMD, so that every chunk of a
// large workload is resident at once (the scalar registers would otherwise
// allow 6 workgroups per CU; the extra ones spill to vector-register lanes,
// not to memory).
__global__ __launch_bounds__(enc_nt(DT)) __attribute__((amdgpu_waves_per_eu(DT == BF16 ? 7 : 1))) void k_analyze(EncArgs a) {
  constexpr int NC = ncoded(DT);
  __shared__ EncShared<DT> sh;
  const int tid = threadIdx.x;
  const uint32_t c = blockIdx.x;
  uint8_t *plan = a.plans + uint64_t(c) * a.plan_stride;
  const uint64_t rec = analyze_chunk<DT, TC>(a, sh, c, plan + plan_fixed(DT));

  // the plan: sizes and offsets, then the code words of coded streams (the
  // counts of a tANS-coded one)
  if (tid == 0) a.sizes[c] = rec;
  if (tid < NC) {
    stg8(plan + 8 * tid, u32x2{uint32_t(sh.bits[tid]), uint32_t(sh.bits[tid] >> 32)});
    stg4(plan + 32 + 4 * tid, uint32_t(sh.sec_off[tid]));
    stg1(plan + 48 + tid, uint32_t(sh.mode[tid]));
    stg1(plan + 52 + tid, uint32_t(sh.aux[tid]));
  }
  for (int p = 0; p < NC; p++) {
    const int A = 1 << kbits(DT, p), mode = sh.mode[p];
    if ((mode == HUFF || mode == GROUP || mode == TANS) && tid < A)
      stg4(plan + 64 + 1024 * p + 4 * tid, sh.enc[p][tid]);
  }
}

// The section of a tANS-coded first stream at sec: head (mode, segment
// count, payload bytes), the presence mask and the counts of the present
// symbols, the segment bit lengths (from the plan), then the payload, each
// segment encoded backwards by one thread at the offset the scan of the
// lengths gives it.  q: the counts (LDS); wtot: LDS scratch.
template <int DT>
__device__ void pack_tans(const uint8_t *src, uint32_t n, bool aligned, int nseg, uint8_t *sec, const uint32_t *q,
                          int A, int k, uint64_t bits, const uint8_t *segbits, TansPack &TP,
                          uint32_t (*wtot)[PACK_NW]) {
  TansEnc<PACK_NT> &T = TP.e;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  int d = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int s = ln + 64 * j;
    d += __popcll(__ballot(s < A && q[s] != 0));
  }
  const uint64_t qoff = 8 + A / 8, soff = qoff + 2ull * d, head = head_bytes_of(TANS, k, nseg, d);
  const uint64_t pay = payload_bytes_of(TANS, k, n, bits);
  if (tid == 0) {
    *reinterpret_cast<uint32_t *>(sec) = uint32_t(TANS) | (uint32_t(nseg) << 16);
    *reinterpret_cast<uint32_t *>(sec + 4) = uint32_t(pay);
  }
  if (tid < A / 8) {
    uint32_t m = 0;
#pragma unroll
    for (int b = 0; b < 8; b++) m |= uint32_t(q[8 * tid + b] != 0) << b;
    sec[8 + tid] = uint8_t(m);
  }
  if (wv == 0) {   // the counts of the present symbols, in symbol order
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) cnt += uint32_t(4 * ln + j < A && q[4 * ln + j] != 0);
    uint32_t idx = wave_incl_scan(cnt) - cnt;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int s = 4 * ln + j;
      if (s < A && q[s] != 0) {
        *reinterpret_cast<uint16_t *>(sec + qoff + 2 * idx) = uint16_t(q[s]);
        idx++;
      }
    }
  }
  for (int j = tid; j < nseg; j += PACK_NT)
    *reinterpret_cast<uint16_t *>(sec + soff + 2 * j) = uint16_t(ldg2(segbits + 2 * j));
  for (uint64_t i = soff + 2ull * nseg + tid; i < head; i += PACK_NT) sec[i] = 0;
  tans_tables<PACK_NT>(q, A, T.tb, nullptr, T.est, T.esym);
  // segment bit offsets: a scan over rows of PACK_NT segments (a chunk of at
  // most 1 MiB has at most 1024 segments per stream)
  constexpr int MAXR = 1024 / PACK_NT;
  uint32_t *pw = reinterpret_cast<uint32_t *>(sec + head);
  int32_t lo[MAXR], hi[MAXR];
  uint32_t carry = 0;
#pragma unroll
  for (int r = 0; r < MAXR; r++) {
    const int j = r * PACK_NT + tid;
    const uint32_t sb = j < nseg ? ldg2(segbits + 2 * j) : 0u;
    const uint32_t incl = wave_incl_scan(sb);
    if (ln == 63) wtot[0][wv] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < PACK_NW; w++) {
      const uint32_t x = wtot[0][w];
      before += w < wv ? x : 0u;
      tot += x;
    }
    __syncthreads();
    lo[r] = int32_t(carry + before + incl - sb);
    hi[r] = lo[r] + int32_t(sb);
    carry += tot;
  }
  // clear the words a segment shares with another (or with the payload's end)
  // and the payload's zero pad, then let every thread's atomic ORs follow.
  // The barrier's workgroup-scope fence is enough: the stores are complete
  // in this XCD's L2 when it passes, and the atomics run there (an
  // agent-scope fence would write the L2 back to memory)
#pragma unroll
  for (int r = 0; r < MAXR; r++) {
    if (r * PACK_NT + tid >= nseg) continue;
    if (lo[r] & 31) stg4(pw + (lo[r] >> 5), 0u);
    if (hi[r] & 31) stg4(pw + ((hi[r] - 1) >> 5), 0u);
  }
  for (uint64_t i = (uint64_t(carry) + 31) / 32 + tid; i < align16(pay) / 4; i += PACK_NT) stg4(pw + i, 0u);
  __syncthreads();
#pragma unroll 1
  for (int r = 0; r < MAXR; r++) {
    const int j = r * PACK_NT + tid;
    if (j >= nseg) continue;
    RingWriter wr(pw, TP.ring[tid], lo[r], hi[r]);
    const uint32_t st = tans_encode_segment<DT>(src, n, aligned, nseg, j, T.esym, T.est,
                                                [&](uint32_t v, uint32_t nb) { wr.put(v, nb); },
                                                [&] { wr.store(); });
    wr.put(st, kTansLog);
    wr.finish();
  }
  __syncthreads();
}

// The record of chunk c at recp: stream heads, raw streams, coded payloads.
// The choice per stream (mode, aux, payload bits, section offset) and the
// code words come from LDS; stage and wtot are LDS scratch of this function.
// PK: some group codes packed exponent pairs (BF16 only)
template <int DT, bool TC, bool PK = false>
__device__ __forceinline__ void pack_chunk(const DevLayout &L, const uint8_t *const *in_ptrs, uint32_t c,
                                           uint8_t *const recp, const uint32_t (*enc)[256], const int *pmode,
                                           const int *paux, const unsigned long long *pbits,
                                           const unsigned long long *psec,
                                           uint32_t (*stage_all)[PackShared<DT>::STAGE],
                                           uint32_t (*wtot)[PACK_NW], uint32_t *rawt,
                                           const uint8_t *segbits, TansPack *tans,
                                           const uint32_t *penc, const uint8_t *prk, bool packed,
                                           const uint32_t *enc2, uint32_t *rawf) {
  constexpr int NC = ncoded(DT), ES = esize(DT), S = segsyms(DT);
  constexpr int VE = 16 / ES;          // elements per 16-byte vector
  constexpr int EPT = S / 64;          // elements per thread per tile (a wave = a segment)
  static_assert(64 * EPT * kMaxLen < 65536, "two segments' bit counts share one 32-bit scan");
  constexpr int NV = EPT / VE;         // vectors per thread per tile
  constexpr int NW = PACK_NW, ENC_NT = PACK_NT, G = PackShared<DT>::G;
  constexpr int STAGE = PackShared<DT>::STAGE;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;

  const int t = find_tensor(L, c);
  const uint64_t e0 = uint64_t(c - L.t_chunk0[t]) * L.chunk_elems;
  const uint64_t rem = L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < L.chunk_elems ? rem : L.chunk_elems);
  const uint8_t *src = in_ptrs[t] + e0 * ES;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const int nseg = int((n + S - 1) / S);
  for (int i = tid; i < 2 * STAGE; i += ENC_NT) stage_all[i / STAGE][i % STAGE] = 0;
  __syncthreads();

  // ------------------------------------------- raw streams
  // Fixed-width values in element order, value bit 0 first; bits past the
  // last element are zero.  For FP32, whose raw streams take whole words in a
  // lane's run of EPT elements (EPT*k = 32), they are written from the tiles
  // of the first coded stream, which read every element anyway: the input is
  // read once.  For 1-byte elements in chunks of whole segments with the
  // exponent coded and the mantissa raw, the exponent's tiles put each strip's
  // mantissa words in LDS and the tile's words go out as rows of 16-byte
  // stores (one row per strip row of the tile's segments).
  // Otherwise (and when no stream is coded) they take one pass of their own
  // here, in element order.
  constexpr bool RSTAGE = PackShared<DT, TC>::RSTAGE;
  constexpr int NWG = NW * G;            // segments per tile
  uint32_t rawmask = 0, tilemask = 0, lmask = 0;
  int firstcoded = -1;
  uint8_t *pwr[NC];
#pragma unroll
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), mode = pmode[p];
    rawmask |= uint32_t(mode == RAW) << p;
    pwr[p] = recp + psec[p] + head_bytes_of(mode, k, nseg);
    if (firstcoded < 0 && (mode == HUFF || mode == GROUP)) firstcoded = p;
  }
  if (firstcoded >= 0) {
#pragma unroll
    for (int p = 0; p < NC; p++)
      if (DT == FP32 && ((rawmask >> p) & 1) && (EPT * kbits(DT, p)) % 32 == 0) tilemask |= 1u << p;
    if (RSTAGE && n % S == 0 && firstcoded == 0 && rawmask == 2u) lmask = 2u;
  }
  static_assert(!RSTAGE || (EPT == 16 && G == 1), "a lane's run is half a strip; one segment per wave");
  // The pass: a lane takes LE consecutive elements per step, LE*k a multiple
  // of 32 for every field width of the dtype, so it writes whole words of
  // every raw stream with no scan; the next step's elements are loaded while
  // this step packs.
  {
    constexpr int LE = DT == FP8 || DT == FP4X2 ? 32 : VE;   // FP8: k = 3 needs 32 elements per 3 words
    constexpr int NQ = LE / VE;                  // 16-byte loads per lane per step
    const uint32_t passmask = rawmask & ~tilemask & ~lmask;
    uint8_t *const *pw = pwr;
    if (passmask) {
      u32x4 nx[NQ];
      auto fetch = [&](uint32_t e) {
        if (aligned && e + LE <= n) {
#pragma unroll
          for (int j = 0; j < NQ; j++) nx[j] = ldg16(src + uint64_t(e + j * VE) * ES);
        }
      };
      fetch(uint32_t(tid) * LE);
      for (uint32_t e = uint32_t(tid) * LE; e < n; e += uint32_t(ENC_NT) * LE) {
        uint32_t w[LE];
        if (aligned && e + LE <= n) {
#pragma unroll
          for (int j = 0; j < NQ; j++) {
            const uint4 xq = make_uint4(nx[j][0], nx[j][1], nx[j][2], nx[j][3]);
#pragma unroll
            for (int i = 0; i < VE; i++) w[j * VE + i] = vec_elem<DT>(xq, i);
          }
        } else {
#pragma unroll
          for (int i = 0; i < LE; i++) w[i] = e + i < n ? load_elem<DT>(src + uint64_t(e + i) * ES) : 0u;
        }
        fetch(e + uint32_t(ENC_NT) * LE);
#pragma unroll
        for (int p = 0; p < NC; p++) {
          if (!((passmask >> p) & 1)) continue;
          constexpr int MAXW = LE * 8 / 32;
          const int k = kbits(DT, p);
          uint32_t wd[MAXW];
#pragma unroll
          for (int x = 0; x < MAXW; x++) wd[x] = 0;
#pragma unroll
          for (int i = 0; i < LE; i++) {
            const uint32_t f = e + i < n ? field_rt<DT>(w[i], p) : 0u;
            const int b = i * k;
            wd[b >> 5] |= f << (b & 31);
            if ((b & 31) + k > 32) wd[(b >> 5) + 1] |= f >> (32 - (b & 31));
          }
          const uint32_t nw = uint32_t((uint64_t(n) * k + 31) / 32), w0 = e / 32 * k + (e % 32) * k / 32;
#pragma unroll
          for (int x = 0; x < MAXW; x++)
            if (x * 32 < LE * k && w0 + x < nw) stg4(pw[p] + 4ull * (w0 + x), wd[x]);
        }
      }
    }
  }

  // -------------------------------------------------------- the record
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k, mode = pmode[p];
    if constexpr (TC) {
      if (mode == TANS) {
        pack_tans<DT>(src, n, aligned, nseg, recp + psec[p], enc[p], A, k, pbits[p], segbits, *tans, wtot);
        // the tables took the tile buffers: clear them for the streams after
        for (int i = tid; i < 2 * STAGE; i += ENC_NT) stage_all[i / STAGE][i % STAGE] = 0;
        __syncthreads();
        continue;
      }
    }
    const uint64_t bits = pbits[p];
    uint8_t *sec = recp + psec[p];
    const uint64_t head = head_bytes_of(mode, k, nseg);
    const uint64_t pay = payload_bytes_of(mode, k, n, bits);
    // stream header, code lengths and the zero pad of the head
    if (tid == 0) {
      *reinterpret_cast<uint32_t *>(sec) =
          uint32_t(mode) | (uint32_t(paux[p]) << 8) | (uint32_t(nseg) << 16);
      *reinterpret_cast<uint32_t *>(sec + 4) = uint32_t(pay);
    }
    uint64_t used = 8;
    if (mode == HUFF) {
      if (tid < A / 2) sec[8 + tid] = uint8_t((enc[p][2 * tid] >> 16) | ((enc[p][2 * tid + 1] >> 16) << 4));
      used += A / 2;
    }
    if (mode == HUFF || mode == GROUP) used += 2ull * nseg;
    for (uint64_t i = used + tid; i < head; i += ENC_NT) sec[i] = 0;
    if (mode == CONST) continue;
    uint32_t *pw = reinterpret_cast<uint32_t *>(sec + head);
    if (mode == RAW) {   // packed above or by the coded stream's tiles; zero the section's pad
      const uint64_t nw = (uint64_t(n) * k + 31) / 32, padw = align16(pay) / 4;
      for (uint64_t i = nw + tid; i < padw; i += ENC_NT) pw[i] = 0;
      continue;
    }
    uint16_t *segt = reinterpret_cast<uint16_t *>(sec + 8 + (mode == HUFF ? A / 2 : 0));
    const bool with_segs = mode != RAW;
    uint64_t tbit = 0;     // stream bits before this tile
    // Huffman-coded streams: tile T holds NW*G consecutive segments; wave w
    // packs segments J = (T*NW + w)*G + g, g < G, whose symbols are the
    // 32-symbol strips J, J + nseg, ... of the chunk; lane l takes symbols
    // [l*EPT, l*EPT + EPT) of each, which lie in one strip.  Raw streams are
    // packed in element order as if cut into segments of S elements.
    const int ntiles = (nseg + NW * G - 1) / (NW * G);
    auto seg_eb = [&](int J) -> uint32_t {  // first element of this lane's run in segment J
      if (with_segs) {
        if (J >= nseg) return n;  // no symbols in this lane
        const uint32_t si = uint32_t(ln) * EPT;
        return 32u * ((si / 32) * uint32_t(nseg) + uint32_t(J)) + si % 32;
      }
      return uint32_t(J) * uint32_t(S) + uint32_t(ln) * EPT;
    };
    // the next tile's 16-byte vectors are loaded one tile ahead
    u32x4 nq[G][NV];
    uint32_t neb[G];
    auto issue = [&](int T) {
#pragma unroll
      for (int g = 0; g < G; g++) {
        neb[g] = seg_eb((T * NW + wv) * G + g);
        if (aligned && neb[g] + EPT <= n) {
#pragma unroll
          for (int j = 0; j < NV; j++) nq[g][j] = ldg16(src + uint64_t(neb[g]) * ES + 16 * j);
        }
      }
    };
    issue(0);
    // FP32 in chunks of whole segments: the raw streams written from these
    // tiles go through the rings
    const bool fring = PackShared<DT, TC>::FRING && p == firstcoded && tilemask && n % S == 0;
    for (int T = 0; T < ntiles; T++) {
      const int buf = T & 1;
      uint32_t *stage = stage_all[buf];
      // Concatenate each run's codes 8 (or, for 4-element runs, 4) at a time
      // without branches: pairs fit 22 bits, quads 44 bits (one u64), two
      // quads 88 bits (lo | hi<<64).
      constexpr int GE = EPT < 8 ? EPT : 8;   // codes per group
      constexpr int NG = EPT / GE;
      uint64_t glo[G][NG];
      uint32_t ghi[G][NG];
      uint32_t gb[G][NG], nb[G];
#pragma unroll
      for (int g = 0; g < G; g++) {
        const uint32_t eb = neb[g];
        const bool vec = aligned && eb + EPT <= n;
        uint32_t w[EPT];
        if constexpr (DT == FP8 || DT == FP4X2) {
          static_assert(NV == 1 && VE == EPT && ES == 1, "a run of 1-byte elements is one 16-byte vector");
          if (!vec) {
            // a run off 16-byte alignment or reaching past the chunk's end:
            // its elements one at a time (zero past the end), placed in the
            // vector as the 16-byte load places them, so everything below
            // reads the vector
            u32x4 q = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < VE; i++) {
              const uint32_t e = eb + uint32_t(i);
              const uint32_t x = e < n ? load_elem<DT>(src + uint64_t(e)) : 0u;
              q[i >> 2] |= x << (8 * (i & 3));
            }
            nq[g][0] = q;
          }
          const uint4 q = make_uint4(nq[g][0][0], nq[g][0][1], nq[g][0][2], nq[g][0][3]);
#pragma unroll
          for (int i = 0; i < VE; i++) w[i] = vec_elem<DT>(q, i);
        } else if (vec) {
#pragma unroll
          for (int j = 0; j < NV; j++) {
            const uint4 q = make_uint4(nq[g][j][0], nq[g][j][1], nq[g][j][2], nq[g][j][3]);
#pragma unroll
            for (int i = 0; i < VE; i++) w[j * VE + i] = vec_elem<DT>(q, i);
          }
        } else {
#pragma unroll
          for (int i = 0; i < EPT; i++)
            w[i] = eb + i < n ? load_elem<DT>(src + uint64_t(eb + i) * ES) : 0;
        }
        nb[g] = 0;
        // elements of this lane's run inside the chunk: the code of every
        // element is read, and those past the end are dropped by a select
        // (no branch per element; their w is 0, a valid table index)
        const uint32_t lim = eb < n ? n - eb : 0u;
        // the raw streams written from these tiles: the run's EPT values are
        // whole words at element eb of each (eb*k is a multiple of 32)
        if (p == firstcoded && tilemask) {
#pragma unroll
          for (int q = 0; q < NC; q++) {
            if (!((tilemask >> q) & 1)) continue;
            const int kq = kbits(DT, q);
            uint64_t bq = 0;   // the run's values, kq bits each (EPT*kq <= 64)
#pragma unroll
            for (int e = 0; e < EPT; e++) {
              const uint32_t f = uint32_t(e) < lim ? field_rt<DT>(w[e], q) : 0u;
              bq |= uint64_t(f) << ((e * kq) & 63);
            }
            const uint32_t nwq = uint32_t((uint64_t(n) * kq + 31) / 32), w0 = eb * kq / 32;
            if constexpr (PackShared<DT, TC>::FRING) {
              if (fring) {
                // word 8J + ln%8 of strip row ln/8, modulo the ring
                static_assert(EPT * 8 == 32 && S == 256, "one word per lane run, 8 strip rows per segment");
                constexpr int FW = PackShared<DT, TC>::FW;
                const int J = (T * NW + wv) * G + g;
                const int qi = __popc(tilemask & ((1u << q) - 1u));
                if (lim > 0) rawf[(qi * 8 + (ln >> 3)) * FW + (8 * J + (ln & 7)) % FW] = uint32_t(bq);
                continue;
              }
            }
#pragma unroll
            for (int x = 0; x < 2; x++)
              if (x * 32 < EPT * kq && lim > 0 && w0 + x < nwq) stg4(pwr[q] + 4ull * (w0 + x), uint32_t(bq >> (32 * x)));
          }
        }
        if constexpr (RSTAGE) if (p == 0 && lmask && lim > 0) {
          // strip ln/2 of this segment, half ln&1: 16 mantissas, 16*KM bits,
          // at 16-bit word KM*(ln&1) of the strip's KM words; every strip is full
          constexpr int KM = kbits(DT, 1);
          static_assert(KM == 2 || KM == 3, "mantissa widths of the 1-byte types");
          uint64_t bq = 0;
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const uint32_t x = nq[g][0][j];
            bq |= uint64_t(mant4<DT>(x)) << (4 * KM * j);
          }
          // the strip of segment s sits at word KM * s of its row, modulo the ring
          constexpr int RW = PackShared<DT, TC>::RW;
          const int s = T * NWG + wv * G + g;
          const int at = (ln >> 1) * (2 * RW) + (s % (RW / KM)) * 2 * KM + (ln & 1) * KM;   // 16-bit words
          uint16_t *rt = reinterpret_cast<uint16_t *>(rawt);
          if constexpr (KM == 2) {
            rawt[at >> 1] = uint32_t(bq);
          } else if (ln & 1) {   // odd half: a 16-bit word, then an aligned 32-bit one
            rt[at] = uint16_t(bq);
            rawt[(at + 1) >> 1] = uint32_t(bq >> 16);
          } else {
            rawt[at >> 1] = uint32_t(bq);
            rt[at + 2] = uint16_t(bq >> 32);
          }
        }
#pragma unroll
        for (int g8 = 0; g8 < NG; g8++) {
          if constexpr ((DT == FP8 || DT == FP4X2) && GE == 8) if (p == 0) {
            // 1-byte elements, first stream: one lookup per two symbols gives
            // their codes joined (the first code's bits, then the second's),
            // the same bits as two single lookups.  Only a run that reaches
            // past the chunk's end takes singles and empties; every other
            // lane skips that branch.
            // elements 8 g8 .. 8 g8 + 7 of the run are words 2 g8, 2 g8 + 1 of
            // its vector; each word's four fields, a byte each, give the
            // indices of its two pairs
            uint32_t ix[4];
#pragma unroll
            for (int h = 0; h < 2; h++) {
              const uint32_t f = field0_4<DT>(nq[g][0][2 * g8 + h]);
              const uint32_t u = f | (f >> 4);     // bytes 0 and 2: x | y << 4
              ix[2 * h] = u & 0xFFu;
              ix[2 * h + 1] = (u >> 16) & 0xFFu;
            }
            if (lim < uint32_t(EPT)) {
#pragma unroll
              for (int j = 0; j < 4; j++) {
                const uint32_t e = uint32_t(g8 * GE + 2 * j);
                ix[j] = e + 1 < lim ? ix[j] : e < lim ? 256u + (ix[j] & 15u) : 272u;
              }
            }
            uint32_t pv[4], pl[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const uint32_t c = enc2[ix[j]];
              pv[j] = c & 0x3FFFFFu;
              pl[j] = c >> 27;
            }
            const uint64_t q0 = uint64_t(pv[0]) | (uint64_t(pv[1]) << pl[0]);
            const uint64_t q1 = uint64_t(pv[2]) | (uint64_t(pv[3]) << pl[2]);
            const uint32_t L0 = pl[0] + pl[1], L1 = pl[2] + pl[3];
            glo[g][g8] = q0 | (q1 << L0);
            ghi[g][g8] = L0 ? uint32_t(q1 >> (64 - L0)) : 0u;
            gb[g][g8] = L0 + L1;
            nb[g] += gb[g][g8];
            continue;
          }
          uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0}, l[8] = {0, 0, 0, 0, 0, 0, 0, 0};
          bool pairs = false;
          if constexpr (DT == BF16 && GE % 2 == 0 && PK) pairs = packed && p == 0;
          if (pairs) {
            // aligned pairs (a run starts at an even place of its strip): a
            // pair of values of F with a pair code is one token, its second
            // slot empty; otherwise two singles (a value past the chunk's end
            // none, a lone last value a single)
#pragma unroll
            for (int j = 0; j < GE / 2; j++) {
              const int e = g8 * GE + 2 * j;
              const uint32_t x = field_rt<DT>(w[e], 0), y = field_rt<DT>(w[e + 1], 0);
              const uint32_t rx = prk[x], ry = prk[y];
              const uint32_t pc = (rx | ry) < 16 ? penc[16 * rx + ry] : 0u;
              const bool tok = uint32_t(e + 1) < lim && (pc >> 16) != 0;
              const uint32_t c0 = tok ? pc : uint32_t(e) < lim ? enc[0][x] : 0u;
              const uint32_t c1 = tok ? 0u : uint32_t(e + 1) < lim ? enc[0][y] : 0u;
              v[2 * j] = c0 & 0xFFFF;
              l[2 * j] = c0 >> 16;
              v[2 * j + 1] = c1 & 0xFFFF;
              l[2 * j + 1] = c1 >> 16;
            }
          } else {
#pragma unroll
            for (int i = 0; i < GE; i++) {
              const int e = g8 * GE + i;
              const uint32_t ce = enc[p][field_rt<DT>(w[e], p)];
              const uint32_t c = uint32_t(e) < lim ? ce : 0u;
              v[i] = c & 0xFFFF;
              l[i] = c >> 16;
            }
          }
          const uint32_t c01 = v[0] | (v[1] << l[0]), l01 = l[0] + l[1];
          const uint32_t c23 = v[2] | (v[3] << l[2]), l23 = l[2] + l[3];
          const uint32_t c45 = v[4] | (v[5] << l[4]), l45 = l[4] + l[5];
          const uint32_t c67 = v[6] | (v[7] << l[6]), l67 = l[6] + l[7];
          const uint64_t q0 = uint64_t(c01) | (uint64_t(c23) << l01);
          const uint64_t q1 = uint64_t(c45) | (uint64_t(c67) << l45);
          const uint32_t L0 = l01 + l23, L1 = l45 + l67;
          glo[g][g8] = q0 | (q1 << L0);
          ghi[g][g8] = L0 ? uint32_t(q1 >> (64 - L0)) : 0u;
          gb[g][g8] = L0 + L1;
          nb[g] += gb[g][g8];
        }
      }
      // issued once this tile's codes are computed, so no later wait for this
      // tile's data also waits for the next tile's loads
      if (T + 1 < ntiles) issue(T + 1);
      // bit offsets: a wave scan per segment, two segments per scan in 16-bit
      // halves (a lane's run codes to at most 16 x 11 bits, a wave's to at
      // most 11264 < 2^16); segments follow each other
      uint32_t incl[G], segtot[G], wsum = 0;
#pragma unroll
      for (int g = 0; g < G; g += 2) {
        if (g + 1 < G) {
          const uint32_t x = wave_incl_scan(nb[g] | (nb[g + 1] << 16));
          incl[g] = x & 0xFFFFu;
          incl[g + 1] = x >> 16;
        } else {
          incl[g] = wave_incl_scan(nb[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; g++) {
        segtot[g] = uint32_t(__builtin_amdgcn_readlane(int(incl[g]), 63));
        wsum += segtot[g];
      }
      if (ln == 0) wtot[buf][wv] = wsum;
      __syncthreads();
      uint32_t woff = 0, ttot = 0;
      for (int q = 0; q < NW; q++) {
        const uint32_t x = wtot[buf][q];
        woff += q < wv ? x : 0;
        ttot += x;
      }
      uint32_t base = uint32_t(tbit & 31) + woff;
#pragma unroll
      for (int g = 0; g < G; g++) {
        const int J = (T * NW + wv) * G + g;
        if (with_segs && ln == 0 && J < nseg) stg2(segt + J, segtot[g]);
        uint32_t start = base + incl[g] - nb[g];
#pragma unroll
        for (int g8 = 0; g8 < NG; g8++) {
          // the 88-bit group shifted to its bit offset covers at most 4 words;
          // ORing zero words is harmless, so no lane branches
          const uint32_t sft = start & 31, wi = start >> 5;
          const uint64_t t0 = glo[g][g8] << sft;
          const uint64_t t1 = (uint64_t(ghi[g][g8]) << sft) | (sft ? glo[g][g8] >> (64 - sft) : 0ull);
          atomicOr(&stage[wi], uint32_t(t0));
          atomicOr(&stage[wi + 1], uint32_t(t0 >> 32));
          atomicOr(&stage[wi + 2], uint32_t(t1));
          atomicOr(&stage[wi + 3], uint32_t(t1 >> 32));
          start += gb[g][g8];
        }
        base += segtot[g];
      }
      if constexpr (RSTAGE) if (p == 0 && lmask) {
        // after a group's last tile and the chunk's last tile: 8 threads per
        // strip row store the row's words from the last store's end up to
        // the last line boundary the group reaches (to the row's end after
        // the last tile); row r's words start at word kq*r*nseg of the stream
        constexpr int RT = PackShared<DT, TC>::RT, RW = PackShared<DT, TC>::RW, q = 1, kq = kbits(DT, 1);
        constexpr int GW = PackShared<DT, TC>::GW;          // a group's words per row
        const bool last = T == ntiles - 1;
        if (T % RT == RT - 1 || last) {
          const uint32_t gi = uint32_t(T / RT), r = uint32_t(tid >> 3), k = uint32_t(tid & 7);
          const uint32_t rowlen = uint32_t(kq) * uint32_t(nseg);
          uint32_t *const dst = reinterpret_cast<uint32_t *>(pwr[q]) + rowlen * r;
          const uint32_t *ring = rawt + r * RW;
          if ((rowlen & 3) == 0 && (reinterpret_cast<uintptr_t>(pwr[q]) & 15) == 0) {
            // rows start 16-byte aligned; phi: the row start's word within its line
            const uint32_t phi = uint32_t(reinterpret_cast<uintptr_t>(dst) >> 2) & 31u;
            auto bound = [&](uint32_t e) {   // the last line boundary at or before word e of the row
              const uint32_t b = (e + phi) & ~31u;
              return b >= phi ? b - phi : 0u;
            };
            const uint32_t f0 = gi == 0 ? 0u : bound(GW * gi);
            const uint32_t f1 = last ? rowlen : bound(GW * (gi + 1));
            for (uint32_t x = f0 + 4 * k; x < f1; x += 32) {
              const uint32_t *sv = ring + x % RW;
              stg16(dst + x, u32x4{sv[0], sv[1], sv[2], sv[3]});
            }
          } else {
            // rows off 16-byte alignment: the group's own words, one at a time
            const uint32_t e = last ? rowlen : GW * (gi + 1);
            for (uint32_t x = GW * gi + k; x < e; x += 8) stg4(dst + x, ring[x % RW]);
          }
        }
      }
      if constexpr (PackShared<DT, TC>::FRING) if (fring) {
        // after every tile: 8 threads per (raw stream, strip row) store the
        // row's whole lines up to the last line boundary the tile reaches
        // (to the row's end after the last tile); row r of a stream starts
        // at word 8*r*nseg
        constexpr int FW = PackShared<DT, TC>::FW, GW = 8 * NWG;
        const uint32_t pr = uint32_t(tid >> 3), k = uint32_t(tid & 7);
        const uint32_t nraw = uint32_t(__popc(tilemask));
        if (pr < 8 * nraw) {
          const uint32_t qi = pr >> 3, r = pr & 7;
          int q = 0;
#pragma unroll
          for (int z = 0, cnt = 0; z < NC; z++) {
            const bool in = (tilemask >> z) & 1;
            q = in && uint32_t(cnt) == qi ? z : q;
            cnt += int(in);
          }
          const bool last = T == ntiles - 1;
          const uint32_t rowlen = 8u * uint32_t(nseg);
          uint32_t *const dst = reinterpret_cast<uint32_t *>(pwr[q]) + rowlen * r;
          const uint32_t *ring = rawf + pr * FW;
          if ((reinterpret_cast<uintptr_t>(pwr[q]) & 15) == 0) {
            const uint32_t phi = uint32_t(reinterpret_cast<uintptr_t>(dst) >> 2) & 31u;
            auto bound = [&](uint32_t e) {   // the last line boundary at or before word e of the row
              const uint32_t b = (e + phi) & ~31u;
              return b >= phi ? b - phi : 0u;
            };
            const uint32_t f0 = T == 0 ? 0u : bound(GW * uint32_t(T));
            const uint32_t f1 = last ? rowlen : bound(GW * uint32_t(T + 1));
            for (uint32_t x = f0 + 4 * k; x < f1; x += 32) {
              const uint32_t *sv = ring + x % FW;
              stg16(dst + x, u32x4{sv[0], sv[1], sv[2], sv[3]});
            }
          } else {
            const uint32_t e = last ? rowlen : GW * uint32_t(T + 1);
            for (uint32_t x = GW * uint32_t(T) + k; x < e; x += 8) stg4(dst + x, ring[x % FW]);
          }
        }
      }
      __syncthreads();
      // store the whole words and clear them for the tile after next; the
      // partial last word moves to word 0 of the next tile's (clear) buffer
      const uint32_t endb = uint32_t(tbit & 31) + ttot;
      const uint32_t nfull = endb >> 5;
      const uint64_t w0 = tbit >> 5;
      for (uint32_t i = tid; i < nfull; i += ENC_NT) {
        stg4(pw + w0 + i, stage[i]);
        stage[i] = 0;
      }
      if (tid == 0) {
        stage_all[buf ^ 1][0] = stage[nfull];
        stage[nfull] = 0;
      }
      tbit += ttot;
    }
    uint32_t carry = 0;   // the partial last word (thread 0 moved it and reads it back)
    if (tid == 0) {
      carry = stage_all[ntiles & 1][0];
      stage_all[ntiles & 1][0] = 0;
    }
    // last partial word and the zero pad of the payload
    const uint64_t words = (tbit + 31) >> 5;
    if (tid == 0 && (tbit & 31)) pw[tbit >> 5] = carry;
    const uint64_t padw = align16(pay) / 4;
    for (uint64_t i = words + tid; i < padw; i += ENC_NT) pw[i] = 0;
  }
}


template <int DT, bool TC>
__device__ __forceinline__ TansPack *tans_of(PackShared<DT, TC> &sh) {
  if constexpr (TC) return &sh.su.tans;
  else return nullptr;
}

// One workgroup per chunk: the record at its directory offset.
template <int DT, bool TC, bool PK = false>
__global__ __launch_bounds__(PACK_NT) void k_pack(PackArgs a) {
  constexpr int NC = ncoded(DT);
  __shared__ PackShared<DT, TC> sh;
  const int tid = threadIdx.x;
  if (a.ctl[0]) return;  // the container did not fit
  // chunks in the reverse of the analysis order: the last chunks analysed
  // are the likeliest still in the 256 MB Infinity Cache
  const uint32_t c = a.L.n_chunks - 1 - blockIdx.x;
  const uint8_t *plan = a.plans + uint64_t(c) * a.plan_stride;
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k, mode = plan[48 + p];
    if (tid < A)
      sh.enc[p][tid] = mode == RAW ? uint32_t(tid) | (uint32_t(k) << 16)
                     : (mode == HUFF || mode == GROUP || mode == TANS) ? ldg4(plan + 64 + 1024 * p + 4 * tid) : 0u;
  }
  bool packed = false;
  if constexpr (DT == BF16 && PK) {
    const int g = plan[52];
    packed = plan[48] == GROUP && a.group_packed && ldg1(a.group_packed + g);
    if (packed) {
      sh.penc[tid] = ldg4(a.group_penc + g * 256 + tid);
      sh.prk[tid] = uint8_t(ldg1(a.group_rank + g * 256 + tid));
    }
  }
  if constexpr (DT == FP8 || DT == FP4X2) {
    // the first stream's joined pair codes, from its single codes
    __syncthreads();
    for (int i = tid; i < 288; i += PACK_NT) {
      const uint32_t cx = sh.enc[0][i & 15], row = uint32_t(i) >> 4;
      const uint32_t cy = row < 16 ? sh.enc[0][row] : 0u;
      const uint32_t lx = cx >> 16, ly = row < 16 ? cy >> 16 : 0u;
      sh.enc2[i] = row < 17 ? ((cx & 0xFFFFu) | ((cy & 0xFFFFu) << lx)) | ((lx + ly) << 27) : 0u;
    }
  }
  if (tid < NC) {
    sh.mode[tid] = plan[48 + tid];
    sh.aux[tid] = plan[52 + tid];
    sh.bits[tid] = *reinterpret_cast<const uint64_t *>(plan + 8 * tid);
    sh.sec_off[tid] = *reinterpret_cast<const uint32_t *>(plan + 32 + 4 * tid);
  }
  const uint64_t *dir = reinterpret_cast<const uint64_t *>(a.out + a.L.off_dir);
  pack_chunk<DT, TC, PK>(a.L, a.in_ptrs, c, a.out + dir[c], sh.enc, sh.mode, sh.aux, sh.bits, sh.sec_off,
                     sh.su.stage, sh.wtot, sh.rawt, plan + plan_fixed(DT), tans_of(sh), sh.penc, sh.prk, packed,
                     sh.enc2, sh.fring);
}

// One workgroup: exclusive scan of the record sizes into the directory, then
// the header, the alignment gaps and the 16-byte zero tail.
__global__ __launch_bounds__(1024) void k_finish(FinishArgs a) {
  __shared__ unsigned long long wsum[16];
  const int tid = threadIdx.x;
  const uint32_t M = a.L.n_chunks;
  const uint32_t per = (M + 1023) / 1024;
  const uint32_t c0 = tid * per, c1 = c0 + per < M ? c0 + per : M;
  // a thread's sizes eight loads at a time (a large model gives each thread
  // dozens; one dependent load per size would make the scan a latency chain)
  unsigned long long s = 0;
  uint32_t c = c0;
  for (; c + 8 <= c1; c += 8) {
    unsigned long long v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = a.sizes[c + i];
#pragma unroll
    for (int i = 0; i < 8; i++) s += v[i];
  }
  for (; c < c1; c++) s += a.sizes[c];
  // block exclusive scan of the per-thread sums
  unsigned long long incl = s;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long t = __shfl_up(incl, o, 64);
    if ((tid & 63) >= o) incl += t;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  unsigned long long before = 0, total = 0;
  for (int w = 0; w < 16; w++) {
    before += w < (tid >> 6) ? wsum[w] : 0;
    total += wsum[w];
  }
  unsigned long long off = a.L.off_records + before + incl - s;
  uint64_t *dir = reinterpret_cast<uint64_t *>(a.out + a.L.off_dir);
  const uint64_t end = a.L.off_records + total;
  const bool fits = end + 16 <= a.cap;
  for (c = c0; c + 8 <= c1; c += 8) {
    unsigned long long v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = a.sizes[c + i];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      stg8(dir + c + i, u32x2{uint32_t(off), uint32_t(off >> 32)});
      off += v[i];
    }
  }
  for (; c < c1; c++) {
    stg8(dir + c, u32x2{uint32_t(off), uint32_t(off >> 32)});
    off += a.sizes[c];
  }
  for (uint32_t i = tid; i < a.hdr_bytes; i += blockDim.x)
    if (i < 56 || i >= 64) stg1(a.out + i, a.hdr[i]);
  const uint64_t dir_end = a.L.off_dir + 8ull * (M + 1);
  const uint64_t raw0 = a.L.T ? a.L.t_raw[0] : a.L.off_records;
  for (uint64_t i = dir_end + tid; i < raw0; i += blockDim.x) stg1(a.out + i, 0);
  for (int t = tid; t < a.L.T; t += blockDim.x) {
    const uint64_t b = a.L.t_raw[t] + rawplane_bytes(a.dtype, a.L.t_n[t]);
    const uint64_t e = t + 1 < a.L.T ? a.L.t_raw[t + 1] : a.L.off_records;
    for (uint64_t i = b; i < e; i++) stg1(a.out + i, 0);
  }
  if (tid == 0) {
    // the only writer of the error word during compression: a store, so the
    // scratch needs no clearing beforehand
    stg4(a.ctl, fits ? 0u : kErrCapacity);
    if (fits) {
      stg8(dir + M, u32x2{uint32_t(end), uint32_t(end >> 32)});
      const uint64_t tot = end + 16;
      stg8(a.out + 56, u32x2{uint32_t(tot), uint32_t(tot >> 32)});
    }
  }
  if (fits && tid < 4) stg4(a.out + end + 4 * tid, 0);
}

uint64_t plan_bytes(int dtype, uint32_t chunk_elems) {
  const uint64_t maxseg = (uint64_t(chunk_elems) + segsyms(dtype) - 1) / segsyms(dtype);
  return align16(plan_fixed(dtype) + 2 * maxseg);
}

hipError_t launch_analyze(int dtype, const EncArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.L.n_chunks == 0) return hipSuccess;
  const dim3 grid(a.L.n_chunks), block(enc_nt(dtype));
  const bool tc = a.coder == CODER_TANS;
  if (dtype == BF16) {
    if (tc) hipExtLaunchKernelGGL((k_analyze<BF16, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_analyze<BF16, false>), grid, block, 0, s, e0, e1, 0, a);
  } else if (dtype == FP32) {
    if (tc) hipExtLaunchKernelGGL((k_analyze<FP32, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_analyze<FP32, false>), grid, block, 0, s, e0, e1, 0, a);
  } else if (dtype == FP8) {
    if (tc) hipExtLaunchKernelGGL((k_analyze<FP8, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_analyze<FP8, false>), grid, block, 0, s, e0, e1, 0, a);
  } else {
    if (tc) hipExtLaunchKernelGGL((k_analyze<FP4X2, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_analyze<FP4X2, false>), grid, block, 0, s, e0, e1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_pack(int dtype, const PackArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.L.n_chunks == 0) return hipSuccess;
  const dim3 grid(a.L.n_chunks), block(PACK_NT);
  const bool tc = a.coder == CODER_TANS;
  if (dtype == BF16) {
    if (tc) hipExtLaunchKernelGGL((k_pack<BF16, true>), grid, block, 0, s, e0, e1, 0, a);
    else if (a.pairs) hipExtLaunchKernelGGL((k_pack<BF16, false, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_pack<BF16, false>), grid, block, 0, s, e0, e1, 0, a);
  } else if (dtype == FP32) {
    if (tc) hipExtLaunchKernelGGL((k_pack<FP32, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_pack<FP32, false>), grid, block, 0, s, e0, e1, 0, a);
  } else if (dtype == FP8) {
    if (tc) hipExtLaunchKernelGGL((k_pack<FP8, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_pack<FP8, false>), grid, block, 0, s, e0, e1, 0, a);
  } else {
    if (tc) hipExtLaunchKernelGGL((k_pack<FP4X2, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((k_pack<FP4X2, false>), grid, block, 0, s, e0, e1, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_finish(const FinishArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL(k_finish, dim3(1), dim3(1024), 0, s, e0, e1, 0, a);
  return hipGetLastError();
}

}  // namespace zn
