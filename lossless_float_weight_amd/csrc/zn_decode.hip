// zn_decode.hip -- the decompression pass for gfx950.
//
// One workgroup of 256 threads (4 wave64s) per chunk.  Reconstruction is
// exact ("NeuralZip: Reusable Setup for Fast Lossless Compression",
// Abstract): every element is reassembled from its coded fields and its
// raw bits (THEORY-599 on ZipNN, per-field compressibility, ZipNN Table II).
//   1. thread 0 walks the chunk record and checks every field against the
//      plan and the buffer bounds;
//   2. each Huffman-coded stream gets an 11-bit multi-symbol table in LDS
//      (up to three code words per lookup), built from the stored code
//      lengths, or copied from the shared group table;
//   3. each lane decodes one segment of one stream -- the per-segment bit
//      lengths give every lane its own start, so segments decode in
//      parallel -- reading its bits through a two-deep 16-byte prefetch;
//   4. decoding runs in rounds of 32 symbols per lane; after each round the
//      workgroup merges the fields staged in LDS with the raw bits and
//      stores whole 16-byte vectors, so stores stay coalesced although every
//      lane works on a different segment.
#include <type_traits>

#include "zn_internal.h"

namespace zn {

constexpr int DEC_NT = 256;
constexpr int RND = 32;        // symbols per lane per round = one strip of its segment
constexpr int STB = 40;        // staging bytes per lane: a strip and up to 5 symbols more
constexpr int RING = 32;       // words of a lane's payload window in LDS: two 64-byte sectors
// The ring is lane-interleaved (word w of thread t at w * DEC_NT + t), so
// lanes that touch different words of their own rings still hit different
// LDS banks.  Staging is STB contiguous bytes per lane: each lookup stores
// its symbols as single bytes at the lane's running position.

// The second stream of FP8 (3-bit mantissas) and FP4 pairs (2-bit mantissa
// pairs) has at most 8 symbols, so no code word is longer than 7 bits and a
// 128-entry table decodes it: with one full table and this one, the LDS of a
// workgroup fits three workgroups per CU.
constexpr int kSmallBits = 7;

template <int DT>
struct DecShared {
  static constexpr int NC = ncoded(DT);
  static constexpr bool SMALL1 = NC == 2;          // stream 1 takes the small table
  static constexpr int NL = SMALL1 ? 1 : NC;       // full tables
  uint32_t lut[NL][kLutSize];
  // 16-byte aligned: the merge reads staged bytes 8 at a time (an unaligned
  // LDS access costs extra cycles)
  alignas(16) union {
    uint16_t t1[kLutSize];
    uint8_t stage[DEC_NT * STB];
    struct {                 // a tANS stream's counts and table construction
      uint32_t q[256];
      int wc[DEC_NT / 64];
      TansBuild<DEC_NT> tb;
    } tq;
  } u;
  alignas(16) uint32_t ring[RING * DEC_NT];
  uint32_t lutm[SMALL1 ? (1 << kSmallBits) : 1];
  uint8_t len[NC][256];
  LutShared ls;
  int mode[NC], aux[NC];
  unsigned long long pay_off[NC], seg_off[NC];
  unsigned long long tq_off;      // a tANS first stream: its presence mask
  int gpacked;                    // the first stream's group codes packed pairs
  uint32_t pay[NC];
  uint32_t wtot[DEC_NT / 64][NC];   // [wave][coded stream index]
  int bad;
};

// Staged bytes [b, b + 8) of thread t (b a multiple of 8).
__device__ __forceinline__ uint64_t stg8(const uint8_t *stage, int b, int t) {
  return *reinterpret_cast<const uint64_t *>(stage + t * STB + b);
}

// (a & m) | (b & ~m) in one instruction (v_bfi_b32); the compiler tends to
// split the two-operand form into three ANDs and an OR.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "s"(m), "v"(a), "v"(b));
  return d;
}

// 8 BF16 values from 8 exponent bytes and 8 sign|fraction bytes: a byte
// permute pairs each value's bytes as [sign|fraction, exponent], then the
// exponent moves down one bit and the sign up to bit 15 of each half.
__device__ __forceinline__ u32x4 merge_bf16(uint64_t E, uint64_t SF) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t e = uint32_t(E >> (32 * h)), s = uint32_t(SF >> (32 * h));
#pragma unroll
    for (int x = 0; x < 2; x++) {
      // bytes [s(2x), e(2x), s(2x+1), e(2x+1)]; e is bytes 4..7 of the pair
      const uint32_t w = __builtin_amdgcn_perm(e, s, x ? 0x07030602u : 0x05010400u);
      o[2 * h + x] = bfi(0x80008000u, w << 8, bfi(0x007F007Fu, w, w >> 1));
    }
  }
  return o;
}

// 4 FP32 values from their four field bytes (exponent; sign and fraction
// bits 22..16; fraction 15..8; fraction 7..0), each field one byte per value:
// a 4x4 byte transpose by permutes gives [f3, f2, f1, f0] per value, then the
// exponent moves down one bit and the sign up to bit 31.
__device__ __forceinline__ u32x4 merge_fp32(uint32_t P0, uint32_t P1, uint32_t P2, uint32_t P3) {
  const uint32_t al = __builtin_amdgcn_perm(P2, P3, 0x05010400u), ah = __builtin_amdgcn_perm(P2, P3, 0x07030602u);
  const uint32_t bl = __builtin_amdgcn_perm(P0, P1, 0x05010400u), bh = __builtin_amdgcn_perm(P0, P1, 0x07030602u);
  const uint32_t X[4] = {__builtin_amdgcn_perm(bl, al, 0x05040100u), __builtin_amdgcn_perm(bl, al, 0x07060302u),
                         __builtin_amdgcn_perm(bh, ah, 0x05040100u), __builtin_amdgcn_perm(bh, ah, 0x07060302u)};
  u32x4 o;
#pragma unroll
  for (int x = 0; x < 4; x++) o[x] = bfi(0x80000000u, X[x] << 8, bfi(0x007FFFFFu, X[x], X[x] >> 1));
  return o;
}

// 8 nibbles (32 bits) -> 8 bytes: a permute spreads the nibble pairs to
// every other byte, then each pair splits across its byte and the next.
__device__ __forceinline__ uint64_t nib_bytes(uint32_t x) {
  const uint32_t lo = __builtin_amdgcn_perm(0u, x, 0x0C010C00u), hi = __builtin_amdgcn_perm(0u, x, 0x0C030C02u);
  return uint64_t((lo | (lo << 4)) & 0x0F0F0F0Fu) | (uint64_t((hi | (hi << 4)) & 0x0F0F0F0Fu) << 32);
}

// 8 values of 3 bits (bits 0..23) -> 8 bytes: pairs of values to bits 0..5
// and 16..21, then each pair splits across its byte and the next.
__device__ __forceinline__ uint64_t tri_bytes(uint32_t x) {
  uint64_t r = 0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t y = x >> (12 * h);
    const uint32_t a = (y & 0x3Fu) | ((y << 10) & 0x3F0000u);
    r |= uint64_t((a | (a << 5)) & 0x07070707u) << (32 * h);
  }
  return r;
}

// 8 values of 2 bits (bits 0..15) -> 8 bytes: the usual bit spread puts each
// value in a nibble of its own, then nib_bytes spreads the nibbles.
__device__ __forceinline__ uint64_t duo_bytes(uint32_t x) {
  x &= 0xFFFFu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return nib_bytes(x);
}

// 4 bytes of FP4 pairs from their exponent pairs (e, a byte each), mantissa
// pairs (m, a byte each) and the 8 sign bits sg (two per byte): each byte is
// m_lo | e_lo << 1 | s_lo << 3 | m_hi << 4 | e_hi << 5 | s_hi << 7.
__device__ __forceinline__ uint32_t merge_fp4x2(uint32_t e, uint32_t m, uint32_t sg) {
  uint32_t t = (sg | (sg << 12)) & 0x000F000Fu;   // sign pairs to their bytes
  t = (t | (t << 6)) & 0x03030303u;
  return (m & 0x01010101u) | ((e & 0x03030303u) << 1) | ((t & 0x01010101u) << 3) |
         ((m & 0x02020202u) << 3) | ((e & 0x0C0C0C0Cu) << 3) | ((t & 0x02020202u) << 6);
}

template <int DT>
__global__ __launch_bounds__(DEC_NT) void k_decode(DecArgs a) {
  constexpr int NC = ncoded(DT), ES = esize(DT), S = segsyms(DT);
  constexpr int VE = 16 / ES;            // elements per 16-byte vector
  __shared__ DecShared<DT> sh;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  const uint32_t c = blockIdx.x;
  // the error word and the chunk's directory entries in one round trip (the
  // directory lies below the records, which the host checked the input holds)
  const uint64_t *dir = reinterpret_cast<const uint64_t *>(a.in + a.L.off_dir);
  const uint32_t ctl0 = a.ctl[0], grouped = a.ctl[1];
  const uint64_t r0 = dir[c], r1 = dir[c + 1];
  if (ctl0) return;  // the header check failed

  const int t = find_tensor(a.L, c);
  const uint64_t e0 = uint64_t(c - a.L.t_chunk0[t]) * a.L.chunk_elems;
  const uint64_t rem = a.L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < a.L.chunk_elems ? rem : a.L.chunk_elems);
  const int nseg = int((n + S - 1) / S);
  uint8_t *dst = a.out_ptrs[t] + e0 * ES;
  const bool oaligned = (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  const uint8_t *in = a.in;
  uint8_t *const sink = reinterpret_cast<uint8_t *>(a.ctl) + kSinkOff;
  const uint8_t *rawp = in + a.L.t_raw[t] + (DT == BF16 ? e0 : DT == FP8 ? e0 / 8 : DT == FP4X2 ? e0 / 4 : 0);

  // The first stream of the record is usually Huffman- or group-coded:
  // its code lengths (Huffman) and segment lengths (at either offset) are
  // loaded with its header, before the walk has read the mode, wherever the
  // record lies inside the input.
  constexpr int A0 = 1 << kbits(DT, 0);
  const bool spec = r0 >= a.L.off_records && (r0 & 15) == 0 &&
                    r0 + 8 + A0 / 2 + 2ull * uint64_t(nseg) <= a.in_bytes;
  uint32_t nib0 = 0, sbh0 = 0, sbg0 = 0;
  if (spec) {
    if (tid < A0) nib0 = ldg1(in + r0 + 8 + (tid >> 1));
    if (tid < nseg) {
      sbh0 = ldg2(in + r0 + 8 + A0 / 2 + 2 * tid);
      sbg0 = ldg2(in + r0 + 8 + 2 * tid);
    }
  }

  // ------------------------------------------------- 1. walk the record
  if (tid == 0) {
    int bad = 0, tsbad = 0;
    sh.gpacked = 0;
    if (r0 < a.L.off_records || r1 < r0 || r1 + 16 > a.in_bytes || (r0 & 15)) bad = 1;
    uint64_t pos = r0;
    for (int p = 0; p < NC && !bad; p++) {
      const int k = kbits(DT, p), A = 1 << k;
      if (pos + 16 > r1) { bad = 1; break; }
      const uint32_t h0 = *reinterpret_cast<const uint32_t *>(in + pos);
      const uint32_t pay = *reinterpret_cast<const uint32_t *>(in + pos + 4);
      const int mode = h0 & 0xFF, aux = (h0 >> 8) & 0xFF, ns = h0 >> 16;
      // tANS codes the exponent stream (the first) only
      if (mode > TANS || ns != nseg || (mode == TANS && p != 0)) { bad = 1; break; }
      int dp = 0;   // tANS: symbols present, from the mask of A bits
      if (mode == TANS) {
        if (pos + 8 + A / 8 > r1) { bad = 1; break; }
        for (int b = 0; b < A / 8; b++) dp += __popc(in[pos + 8 + b]);
      }
      const uint64_t head = head_bytes_of(mode, k, nseg, dp);
      if (pos + head + align16(pay) > r1) { bad = 1; break; }
      if (mode == TANS && (aux != 0 || pay == 0 || (pay & 3))) bad = 1;
      if (mode == CONST && (aux >= A || pay != 0)) bad = 1;
      if (mode == RAW && (aux != 0 || pay != (uint64_t(n) * k + 7) / 8)) bad = 1;
      if (mode == HUFF && (aux != 0 || pay == 0 || (pay & 3))) bad = 1;
      // a group code only for the first stream of a container made with
      // groups; a group id the tableset lacks is a tableset mismatch, and an
      // empty group (its decode table is all zero) has no code at all
      if (mode == GROUP && (p != 0 || !grouped || pay == 0 || (pay & 3))) bad = 1;
      if (mode == GROUP && !bad && aux >= a.K) tsbad = 1;
      if (mode == GROUP && !bad && !tsbad && ldg4(a.group_lut + size_t(aux) * kLutSize) == 0) bad = 1;
      if (mode == GROUP && !bad && !tsbad) sh.gpacked = a.group_packed ? ldg1(a.group_packed + aux) : 0;
      if (tsbad) break;
      sh.mode[p] = mode;
      sh.aux[p] = aux;
      sh.pay[p] = pay;
      sh.pay_off[p] = pos + head;
      sh.seg_off[p] = pos + 8 + (mode == HUFF ? A / 2 : 0) + (mode == TANS ? A / 8 + 2 * dp : 0);
      if (mode == TANS) sh.tq_off = pos + 8;
      pos += head + align16(pay);
    }
    if (!bad && !tsbad && pos != r1) bad = 1;
    sh.bad = bad ? int(kErrCorrupt) : tsbad ? int(kErrTableset) : 0;
  }
  __syncthreads();
  if (sh.bad) {
    if (tid == 0) atomicOr(&a.ctl[0], uint32_t(sh.bad));
    return;
  }

  // ------------------------------------------------ 3. lanes and rounds
  // Lanes decode only the Huffman- or group-coded streams; raw and constant
  // streams need no decoding and the merge reads them straight from the
  // record.  With ncc coded streams, SPW = 64, 32 or 16 lanes of each wave
  // take one coded stream each (a template per SPW; the branch below is
  // uniform per workgroup).
  // The coded streams as a bit mask (no array indexed by a lane-dependent
  // value, which the compiler would place in scratch memory): the ci-th coded
  // stream is the ci-th set bit, and stream p is coded stream number
  // popcount(codedm below p).
  int ncc = 0, codedm = 0, rawm = 0, constm = 0;
#pragma unroll
  for (int p = 0; p < NC; p++) {
    const bool cod = sh.mode[p] == HUFF || sh.mode[p] == GROUP || sh.mode[p] == TANS;
    codedm |= int(cod) << p;
    ncc += int(cod);
    rawm |= int(sh.mode[p] == RAW) << p;
    constm |= int(sh.mode[p] == CONST) << p;
  }
  auto nth_coded = [&](int k) {   // the stream of coded-stream number k (0 if none)
    int r = 0, cnt = 0;
#pragma unroll
    for (int q = 0; q < NC; q++) {
      const bool isc = (codedm >> q) & 1;
      r = isc && cnt == k ? q : r;
      cnt += int(isc);
    }
    return r;
  };
  auto cidx = [&](int p) { return __popc(uint32_t(codedm) & ((1u << p) - 1u)); };
  // Lanes per coded stream, as the dispatch at the end chooses it: all
  // coded streams share each wave; FP32 with a coded exponent and raw or
  // constant fraction bytes gives the exponent every lane; any other FP32
  // mix takes 16 lanes per stream.
  const int spw = ncc == NC ? 64 / NC
                  : NC <= 2 ? 64
                  : ncc == 1 && (rawm == 14 || (rawm == 2 && constm == 12)) ? 64 : 16;
  // The first segment length of this lane, loaded before the tables are
  // built so that its latency overlaps the build.
  uint32_t sbits0 = 0;
  {
    const int ci = ln / spw, sj = wv * spw + ln % spw;
    if (ci < ncc && sj < nseg) {
      const int pc = nth_coded(ci);
      if (spec && pc == 0 && sj == tid && sh.mode[0] != TANS) sbits0 = sh.mode[0] == HUFF ? sbh0 : sbg0;
      else sbits0 = ldg2(in + sh.seg_off[pc] + 2 * sj);
    }
  }
  // ---------------------------------------------------------- 2. tables
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k, mode = sh.mode[p];
    if (mode == HUFF) {
      const uint8_t *nib = in + sh.seg_off[p] - A / 2;
      if (tid < A) {
        const uint32_t x = p == 0 && spec ? nib0 : ldg1(nib + (tid >> 1));
        sh.len[p][tid] = (x >> ((tid & 1) * 4)) & 15;
      }
      __syncthreads();
      bool ok;
      if constexpr (DecShared<DT>::SMALL1) {
        ok = p == 1 ? build_lut<DEC_NT, kSmallBits>(sh.len[p], A, sh.lutm, sh.u.t1, sh.ls)
                    : build_lut<DEC_NT>(sh.len[p], A, sh.lut[0], sh.u.t1, sh.ls);
      } else {
        ok = build_lut<DEC_NT>(sh.len[p], A, sh.lut[p], sh.u.t1, sh.ls);
      }
      if (!ok) {
        if (tid == 0) atomicOr(&a.ctl[0], kErrCorrupt);
        return;
      }
    } else if (mode == GROUP) {
      const uint32_t *gl = a.group_lut + size_t(sh.aux[p]) * kLutSize;
      for (int i = tid; i < kLutSize; i += DEC_NT) sh.lut[DecShared<DT>::SMALL1 ? 0 : p][i] = ldg4(gl + i);
      if (tid < A) sh.len[p][tid] = ldg1(a.group_len + sh.aux[p] * 256 + tid);
    } else if (mode == TANS) {
      // the counts: the mask's present symbols take the stored values in
      // symbol order, each at least 1; the table needs their sum to be 2^11
      auto &T = sh.u.tq;
      const uint8_t *mk = in + sh.tq_off;
      const bool pres = tid < A && ((ldg1(mk + (tid >> 3)) >> (tid & 7)) & 1);
      const uint64_t m = __ballot(pres);
      if (ln == 0) T.wc[wv] = __popcll(m);
      __syncthreads();
      uint32_t idx = uint32_t(__popcll(m & lanemask_lt()));
      for (int w = 0; w < wv; w++) idx += uint32_t(T.wc[w]);
      const uint32_t qv = pres ? ldg2(mk + A / 8 + 2 * idx) : 0u;
      if (tid < A) T.q[tid] = qv;
      const int zero = __syncthreads_or(pres && qv == 0);
      const bool ok = tans_tables<DEC_NT>(T.q, A, T.tb, sh.lut[0], nullptr, nullptr);
      if (zero || !ok) {
        if (tid == 0) atomicOr(&a.ctl[0], kErrCorrupt);
        return;
      }
    }
  }
  __syncthreads();

  // Fields of the raw streams for one 16-byte output vector of VE elements
  // starting at element ev (< n): k = 8 gives VE bytes, k = 4 VE nibbles,
  // k = 3 a 3*VE-bit run, k = 2 a 2*VE-bit word.  Every read stays inside the stream's payload, or
  // at most 4 bytes past it where the record or the container tail follows
  // (the record walk checked that the container holds them).
  // payload bases as wave-uniform values, so loads take a scalar base and a
  // 32-bit lane offset
  const uint8_t *payu[NC];
#pragma unroll
  for (int p = 0; p < NC; p++) {
    const uint64_t po = sh.pay_off[p];
    payu[p] = in + ((uint64_t(__builtin_amdgcn_readfirstlane(uint32_t(po >> 32))) << 32) |
                    __builtin_amdgcn_readfirstlane(uint32_t(po)));
  }
  auto raw_field = [&](int p, uint32_t ev) -> uint64_t {
    const uint8_t *pay = payu[p];
    const int k = kbits(DT, p);
    if (k == 8) {
      if constexpr (VE == 8) { const u32x2 x = ldg8(pay + ev); return x[0] | (uint64_t(x[1]) << 32); }
      else if constexpr (VE == 4) return ldg4(pay + ev);
      else return 0;
    }
    if (k == 4) { const u32x2 x = ldg8(pay + ev / 2); return x[0] | (uint64_t(x[1]) << 32); }
    if (k == 2) return ldg4(pay + ev / 4);   // ev is a multiple of 16: a whole word
    const uint32_t b = ev * 3, w0 = b >> 5;   // ev is a multiple of 16: b & 31 is 0 or 16
    const uint64_t x = ldg4(pay + 4 * w0) | (uint64_t(ldg4(pay + 4 * w0 + 4)) << 32);
    return x >> (b & 31);
  };
  // a constant stream's byte in every byte lane
  auto cfield = [&](int p) -> uint64_t { return 0x0101010101010101ull * uint64_t(sh.aux[p]); };

  int bad = 0;
  auto path = [&](auto spw_c, auto rawf_c, auto allc_c, auto rawm_c, auto constm_c, auto tans_c) {
    constexpr int SPW = decltype(spw_c)::value;   // lanes per coded stream per wave
    constexpr bool TANS0 = decltype(tans_c)::value; // the first stream is tANS-coded
    constexpr bool RAWF = decltype(rawf_c)::value; // some stream is stored raw
    constexpr bool ALLC = decltype(allc_c)::value; // every stream is coded
    // RAWM != 0: stream p is raw if bit p of RAWM is set, constant if bit p
    // of CONSTM is, coded otherwise -- known here, so only the raw streams'
    // fields are loaded and held and no mode is tested per vector
    constexpr int RAWM = decltype(rawm_c)::value;
    constexpr int CONSTM = decltype(constm_c)::value;
    if (spw != SPW) { bad = 1; return; }   // the layout sbits0 was loaded for
    constexpr int GS = 4 * SPW;                   // segments per coded stream per group
    constexpr int VPS = RND * ES / 16;            // output vectors per strip
    constexpr int NVL = SPW * VPS / 64;           // output vectors per lane per round
    // Lane (wave wv, lane ln) decodes coded stream ci = ln / SPW, segment slot
    // wv*SPW + ln%SPW.  Round r decodes strip r*nseg + j of every segment j,
    // so one round of a wave covers SPW consecutive strips: a contiguous
    // block of the output.
    const int ci = ln / SPW, slot = wv * SPW + ln % SPW;
    const bool coded = ci < ncc;
    const int p = coded ? nth_coded(ci) : 0;
    const uint8_t *pay = in + sh.pay_off[p];
    const uint32_t paybytes = sh.pay[p];
    const uint32_t ngroups = (paybytes + 15) / 16;
    constexpr bool SMALL1 = DecShared<DT>::SMALL1;
    const bool small = SMALL1 && p == 1;
    const uint32_t *lut = small ? sh.lutm : sh.lut[SMALL1 ? 0 : p];
    // byte offset of the entry of the window's next bits (W = window << 2)
    const uint32_t wmask = small ? ((1u << kSmallBits) - 1) << 2 : uint32_t(kLutSize - 1) << 2;
    uint8_t *sb = sh.u.stage + tid * STB;   // this lane's staged symbols
    uint32_t *rp = sh.ring + tid;       // ring word w of this lane: rp[w * DEC_NT]
    const int t0 = wv * 64;             // first thread of this wave
    uint32_t seg_carry = 0;
    const uint32_t nstrips = (n + RND - 1) / RND;
    const int G = (nseg + GS - 1) / GS;
    for (int g = 0; g < G; g++) {
      const int sj = g * GS + slot;
      const bool live = sj < nseg;
      // start bit of the segment: scan of the stored segment bit lengths
      uint32_t sbits = sbits0;
      if (g > 0 && coded && live) sbits = ldg2(in + sh.seg_off[p] + 2 * sj);
      const uint32_t incl = wave_incl_scan(sbits);
      const int first = ci * SPW;
      // every lane takes part in the shuffle: a lane left out of it by a
      // branch returns 0 to the lanes reading from it
      const uint32_t wprev = __shfl(incl, (first + 63) & 63, 64);
      const uint32_t wbase = first > 0 ? wprev : 0;
      const uint32_t wlast = __shfl(incl, (first + SPW - 1) & 63, 64);
      if (coded && ln == first) sh.wtot[wv][ci] = wlast - wbase;
      __syncthreads();
      uint32_t before = 0, gtot = 0;
      if (coded) {
#pragma unroll
        for (int q = 0; q < DEC_NT / 64; q++) {
          const uint32_t x = sh.wtot[q][ci];
          before += q < wv ? x : 0;
          gtot += x;
        }
      }
      const uint32_t b0 = seg_carry + before + (incl - sbits - wbase);
      seg_carry += gtot;
      __syncthreads();

      // Bit reader: a window of nb bits (LSB-first) refilled one word at a
      // time from the lane's ring of payload words in LDS, kept shifted up
      // by two (W = window << 2) so that W & wmask is the byte offset of
      // the table entry of its next 11 bits (7 for the small table).  The ring holds two 64-byte
      // sectors of the payload, aligned in memory so that every sector is
      // one HBM burst read once; a sector is loaded one round before it can
      // be needed.  Word positions count from the aligned base.
      uint64_t W = 0;
      int nb = 0;
      const uintptr_t pa = reinterpret_cast<uintptr_t>(pay);
      const uint8_t *pay64 = pay - (pa & 63);       // inside the container: pay is past the header
      const uint32_t adj = uint32_t(pa & 63) / 4;   // payload word 0 is window word adj
      const uint32_t glast = adj / 4 + ngroups - 1; // last 16-byte group holding payload
      uint32_t wpos = 0, nsec = 0, pre = 0;         // next word to read, next sector to fetch
      uint32_t slast = 0;                           // last sector holding bits of the segment
      u32x4 ps0 = {0, 0, 0, 0}, ps1 = ps0, ps2 = ps0, ps3 = ps0;
      // The segment's last sector, when it is not among the first two: it is
      // the next segment's first, which the neighbouring lane loads now, so it
      // is loaded now as well (one read of the line) and held until needed,
      // rather than read again from memory at the segment's end.
      u32x4 hl0 = ps0, hl1 = ps0, hl2 = ps0, hl3 = ps0;
      bool hold = false;
      bool pend = false;
      // 16-byte group gi of the window; groups past the payload read its last one
      auto grp = [&](uint32_t gi) { return ldg16(pay64 + 16ull * (gi < glast ? gi : glast)); };
      auto put_sector = [&](uint32_t sc, const u32x4 &x0, const u32x4 &x1, const u32x4 &x2,
                            const u32x4 &x3) {
        uint32_t *q = rp + (sc & 1) * 16 * DEC_NT;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
          q[kk * DEC_NT] = x0[kk];
          q[(4 + kk) * DEC_NT] = x1[kk];
          q[(8 + kk) * DEC_NT] = x2[kk];
          q[(12 + kk) * DEC_NT] = x3[kk];
        }
      };
      if (coded && live) {
        const uint32_t w0 = (b0 >> 5) + adj, s0 = w0 >> 4;
        // No sector past the one holding the segment's last bit is loaded:
        // it belongs to the next segment, whose lane read it long ago.
        slast = (((b0 + sbits - 1) >> 5) + adj) >> 4;
        const uint32_t s1 = s0 + 1 <= slast ? s0 + 1 : s0;
        const u32x4 a0 = grp(4 * s0), a1 = grp(4 * s0 + 1), a2 = grp(4 * s0 + 2), a3 = grp(4 * s0 + 3);
        const u32x4 a4 = grp(4 * s1), a5 = grp(4 * s1 + 1), a6 = grp(4 * s1 + 2), a7 = grp(4 * s1 + 3);
        hold = slast > s0 + 1;
        if (hold) {
          hl0 = grp(4 * slast);
          hl1 = grp(4 * slast + 1);
          hl2 = grp(4 * slast + 2);
          hl3 = grp(4 * slast + 3);
        }
        put_sector(s0, a0, a1, a2, a3);
        put_sector(s0 + 1, a4, a5, a6, a7);
        // the held sector's loads complete here, with the first two, so no
        // wait inside the rounds is for them
        asm volatile("" ::"v"(hl0[0]), "v"(hl0[1]), "v"(hl0[2]), "v"(hl0[3]), "v"(hl1[0]), "v"(hl1[1]),
                     "v"(hl1[2]), "v"(hl1[3]), "v"(hl2[0]), "v"(hl2[1]), "v"(hl2[2]), "v"(hl2[3]),
                     "v"(hl3[0]), "v"(hl3[1]), "v"(hl3[2]), "v"(hl3[3]));
        nsec = s0 + 2;
        W = uint64_t(rp[(w0 & (RING - 1)) * DEC_NT] >> (b0 & 31)) << 2;
        wpos = w0 + 1;
        nb = 32 - int(b0 & 31);
      }
      int ov = 0;         // symbols of the next strip decoded early (staged words 8, 9)
      uint32_t tx = 0;    // tANS: the lane's state minus 2^11
      uint64_t cur = 0;   // staged bytes not yet stored whole: those of the word at a, then the next
      // Raw bits and raw-stream fields merged by this lane in round r: the
      // same loads every round (an empty vector reads element 0 and is
      // ignored; r = -1, after the last round, reads element 0 everywhere),
      // so no wait has to drain the stores in flight.  A partial
      // last vector stays inside the always-raw plane, whose size is padded
      // to 16 bytes: BF16 vectors start at multiples of 8 bytes, FP8 sign
      // words at multiples of 2, FP4 sign words at multiples of 4.
      using FT = std::conditional_t<ES == 4, uint32_t, uint64_t>;  // VE raw-stream fields
      struct RawIn { uint64_t plane[NVL]; FT f[NC][NVL]; };
      auto load_raw = [&](int r, RawIn &rv) {
#pragma unroll
        for (int i = 0; i < NVL; i++) {
          const int v = ln + 64 * i, sl = v / VPS, part = v % VPS;
          const int sjv = g * GS + wv * SPW + sl;
          const uint32_t ev0 = (uint32_t(r) * nseg + sjv) * RND + part * VE;
          const uint32_t ev = r >= 0 && sjv < nseg && ev0 < n ? ev0 : 0;
          if constexpr (DT == BF16) {
            const u32x2 x = ldg8s(rawp + ev);
            rv.plane[i] = x[0] | (uint64_t(x[1]) << 32);
          } else if constexpr (DT == FP8) {
            rv.plane[i] = ldg2(rawp + ev / 8);
          } else if constexpr (DT == FP4X2) {
            rv.plane[i] = ldg4(rawp + ev / 4);    // two sign bits per element
          } else {
            rv.plane[i] = 0;
          }
          if constexpr (RAWM != 0) {
#pragma unroll
            for (int q = 0; q < NC; q++)
              if ((RAWM >> q) & 1) rv.f[q][i] = FT(raw_field(q, ev));
          } else if constexpr (RAWF) {
#pragma unroll
            for (int q = 0; q < NC; q++) rv.f[q][i] = sh.mode[q] == RAW ? FT(raw_field(q, ev)) : FT(0);
          }
          if constexpr (NVL > 4) __builtin_amdgcn_sched_barrier(0);   // addresses of one vector live at a time
        }
      };
      constexpr int NR = S / RND;   // rounds, an even number
      static_assert(NR % 2 == 0, "rounds come in pairs");
      RawIn rawA, rawB;
      load_raw(0, rawA);
      // One round; the raw inputs of the next round load into nxt while this
      // one decodes (the loop below alternates two register sets, so no copy
      // makes the compiler wait for loads in flight).
      auto round = [&](int r, const RawIn &rawv, RawIn &nxt) {
        load_raw(r + 1 < NR ? r + 1 : -1, nxt);  // the last round loads one line: same count
        const uint32_t q = uint32_t(r) * nseg + sj;   // this lane's strip
        const int lim = coded && live && q < nstrips ? int(min(uint32_t(RND), n - q * RND)) : 0;
        const bool last = live && q < nstrips && q + nseg >= nstrips;
        // the sector fetched last round enters the ring
        if (pend) {
          put_sector(nsec, ps0, ps1, ps2, ps3);
          nsec++;
          pend = false;
        }
        if (TANS0 && p == 0 && lim > 0) {
          // tANS: one table step per symbol.  The segment opens with the
          // encoder's final state (11 bits); each step reads the state's
          // entry (symbol, bit count, base of the next state) and adds the
          // next bits to the base.  The window takes a word whenever fewer
          // than 22 bits remain (two steps need at most 22), so, as for the
          // Huffman lanes, a round reads at most 12 words.  Symbols are staged
          // four to a word at bytes 0..lim of the lane's staging area.
          const uint32_t abase = uint32_t(tid * STB);
          uint32_t *const stw = reinterpret_cast<uint32_t *>(sh.u.stage);
          pre = rp[__builtin_amdgcn_ubfe(wpos, 0, 5) * DEC_NT];
          auto refill = [&](int below) {
            const bool need = nb < below;
            W |= uint64_t(need ? pre : 0u) << (nb + 2);
            nb += need ? 32 : 0;
            wpos += need ? 1u : 0u;
            pre = rp[__builtin_amdgcn_ubfe(wpos, 0, 5) * DEC_NT];
          };
          if (r == 0) {
            refill(kTansLog);
            tx = (uint32_t(W) >> 2) & (kTansStates - 1);
            W >>= kTansLog;
            nb -= kTansLog;
          }
          auto tstep = [&]() -> uint32_t {
            const uint32_t e = lut[tx];
            const uint32_t kb = (e >> 8) & 15u;
            tx = (e >> 12) + ((uint32_t(W) >> 2) & ((1u << kb) - 1u));
            W >>= kb;
            nb -= int(kb);
            return e & 0xFFu;
          };
          uint32_t word = 0;
          for (int i = 0; i < lim; i += 2) {
            refill(22);
            word |= tstep() << (8 * (i & 3));
            if (i + 1 < lim) word |= tstep() << (8 * ((i + 1) & 3));
            if ((i & 3) == 2 || i + 2 >= lim) {
              stw[(abase + uint32_t(i & ~3)) >> 2] = word;
              word = 0;
            }
          }
          if (last) {
            // exact end: the stored bit length used up, back in state 2^11
            const uint64_t bpos = uint64_t(wpos - adj) * 32 - uint32_t(nb);
            if (bpos != uint64_t(b0) + sbits || tx != 0) bad = 1;
          } else if (((wpos + 11) >> 4) >= nsec && nsec <= slast) {
            if (hold && nsec == slast) {
              ps0 = hl0;
              ps1 = hl1;
              ps2 = hl2;
              ps3 = hl3;
            } else {
              ps0 = grp(4 * nsec);
              ps1 = grp(4 * nsec + 1);
              ps2 = grp(4 * nsec + 2);
              ps3 = grp(4 * nsec + 3);
            }
            pend = true;
          }
        } else if (lim > 0) {
          // Each lookup appends its (up to three) symbols, one byte each, to
          // the lane's staged bytes: they join the pending bytes of the
          // current word in cur, which is stored whole and aligned (single
          // bytes would each cost the LDS a partial-word write); a word that
          // fills moves the rest of cur down.  The window is refilled, without
          // branches, with 32 bits whenever fewer than 30 remain: enough for
          // the two lookups of an iteration (at most 22 bits), and the word
          // lands at bit nb + 2 <= 31 of W, so nothing falls off its top.
          if (ov) {  // symbols of this strip decoded last round: bytes 32.. -> 0..
            uint32_t *sw = reinterpret_cast<uint32_t *>(sb);
            const uint32_t c8 = sw[8], c9 = sw[9];
            sw[0] = c8;
            sw[1] = c9;
          }
          // a: stage byte of the next symbol; nbk + 64 a == nb + 2 at all
          // times, so a lookup updates both with its low byte (bits used +
          // 64 x symbols) and the refill test needs one multiply-add.
          const uint32_t abase = uint32_t(tid * STB);
          uint32_t a = abase + uint32_t(ov);
          const uint32_t alim = abase + uint32_t(lim);
          uint32_t nbk = uint32_t(nb + 2) - (a << 6);
          pre = rp[__builtin_amdgcn_ubfe(wpos, 0, 5) * DEC_NT];
          const uint8_t *lutb = reinterpret_cast<const uint8_t *>(lut);
          uint32_t *const stw = reinterpret_cast<uint32_t *>(sh.u.stage);   // abase is a multiple of 8
          auto step = [&]() -> uint32_t {
            const uint32_t e = *reinterpret_cast<const uint32_t *>(lutb + (uint32_t(W) & wmask));
            cur |= uint64_t(e >> 8) << ((a & 3) * 8);   // unused symbol bytes of an entry are zero
            stw[a >> 2] = uint32_t(cur);
            const uint32_t an = a + ((e >> 6) & 3);
            cur = (an ^ a) > 3 ? cur >> 32 : cur;
            a = an;
            W >>= (e & 63);
            nbk -= e & 0xFF;
            return e;
          };
          // packed pairs take one token per table entry: the staging place
          // after the first lookup of the last pair, and the second's entry,
          // tell the exact end of the segment
          uint32_t a1 = a, e2 = 0;
          while (a < alim) {
            const uint32_t t = nbk + (a << 6);   // nb + 2
            const bool need = t < 32;
            W |= uint64_t(need ? pre : 0u) << t;
            nbk += need ? 32u : 0u;
            wpos += need ? 1u : 0u;
            pre = rp[__builtin_amdgcn_ubfe(wpos, 0, 5) * DEC_NT];
            step();
            a1 = a;
            e2 = step();
          }
          stw[a >> 2] = uint32_t(cur);   // the last, partial word
          const int pos = int(a - abase);
          nb = int(nbk + (a << 6)) - 2;
          ov = pos - lim;   // at most 5: the loop stops 2 lookups of 3 symbols past lim - 1
          if (last) {
            // exact end: the segment must use exactly its stored bit length
            uint64_t bpos = uint64_t(wpos - adj) * 32 - uint32_t(nb);
            if (p == 0 && sh.gpacked) {
              // tokens of packed pairs: past the end may lie only the whole
              // token of the last lookup, after a first lookup that ended
              // exactly there (a pair across the end is not a valid stream)
              if (ov > 0) {
                if (a1 == alim && uint32_t(ov) == ((e2 >> 6) & 3)) bpos -= e2 & 63;
                else bad = 1;
              }
            } else {
              for (int x = 0; x < ov; x++) {
                const int bb = lim + x;
                bpos -= sh.len[p][sb[bb]];
              }
            }
            if (bpos != uint64_t(b0) + sbits) bad = 1;
            ov = 0;
            cur = 0;
          } else if (((wpos + 11) >> 4) >= nsec && nsec <= slast) {
            // lim == RND here.  The next round reads at most 32 lookups (352
            // bits); the window now holds at least 8 bits and takes a word
            // only while it holds fewer than 30, so at most 12 words
            // [wpos, wpos + 12): at most one sector past those in the ring,
            // whose slot held a sector before wpos's.
            if (hold && nsec == slast) {
              ps0 = hl0;
              ps1 = hl1;
              ps2 = hl2;
              ps3 = hl3;
            } else {
              ps0 = grp(4 * nsec);
              ps1 = grp(4 * nsec + 1);
              ps2 = grp(4 * nsec + 2);
              ps3 = grp(4 * nsec + 3);
            }
            pend = true;
          }
        }
        wave_lds_sync();
        // merge: vector v of this wave covers VE elements of slot v / VPS
        auto vec = [&](int i, uint32_t &ev, bool &valid) -> u32x4 {
          const int v = ln + 64 * i, sl = v / VPS, part = v % VPS;
          const int sjv = g * GS + wv * SPW + sl;
          ev = (uint32_t(r) * nseg + sjv) * RND + part * VE;
          valid = sjv < nseg && ev < n;
          // staged bytes of coded stream pp for this vector (VE bytes)
          auto staged = [&](int pp, int h) -> uint64_t {
            const int th = t0 + cidx(pp) * SPW + sl;
            if constexpr (ES == 2) return stg8(sh.u.stage, 8 * part, th);
            else if constexpr (ES == 4) return *reinterpret_cast<const uint32_t *>(sh.u.stage + th * STB + 4 * part);
            else return stg8(sh.u.stage, 16 * part + 8 * h, th);
          };
          auto fieldv = [&](int pp, int h) -> uint64_t {   // h: 8-byte half (FP8)
            if constexpr (ALLC) {
              return staged(pp, h);
            } else if constexpr (RAWM != 0) {
              if ((CONSTM >> pp) & 1) return cfield(pp);
              return ((RAWM >> pp) & 1) ? uint64_t(rawv.f[pp][i]) : staged(pp, h);
            } else {
              const int md = sh.mode[pp];
              if (md == CONST) return cfield(pp);
              if (md != RAW || !RAWF) return staged(pp, h);
              return rawv.f[pp][i];
            }
          };
          u32x4 o;
          if constexpr (DT == BF16) {
            o = merge_bf16(fieldv(0, 0), rawv.plane[i]);
          } else if constexpr (DT == FP32) {
            o = merge_fp32(uint32_t(fieldv(0, 0)), uint32_t(fieldv(1, 0)), uint32_t(fieldv(2, 0)),
                           uint32_t(fieldv(3, 0)));
          } else if constexpr (DT == FP4X2) {
            // exponent pairs and mantissa pairs of the 16 elements as bytes
            uint64_t Ev[2], Mv[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
              const bool r0 = RAWM != 0 ? (RAWM & 1) != 0 : !ALLC && RAWF && sh.mode[0] == RAW;
              const bool r1 = RAWM != 0 ? (RAWM & 2) != 0 : !ALLC && RAWF && sh.mode[1] == RAW;
              if (r0) Ev[h] = nib_bytes(uint32_t(rawv.f[0][i] >> (32 * h)));
              else Ev[h] = fieldv(0, h);
              if (r1) Mv[h] = duo_bytes(uint32_t(rawv.f[1][i] >> (16 * h)));
              else Mv[h] = fieldv(1, h);
            }
#pragma unroll
            for (int x = 0; x < 4; x++)
              o[x] = merge_fp4x2(uint32_t(Ev[x >> 1] >> (32 * (x & 1))), uint32_t(Mv[x >> 1] >> (32 * (x & 1))),
                                 uint32_t(rawv.plane[i] >> (8 * x)) & 0xFFu);
          } else {
            // E4 and M3 of the 16 elements as bytes, from whichever source
            uint64_t Ev[2], Mv[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
              const bool r0 = RAWM != 0 ? (RAWM & 1) != 0 : !ALLC && RAWF && sh.mode[0] == RAW;
              const bool r1 = RAWM != 0 ? (RAWM & 2) != 0 : !ALLC && RAWF && sh.mode[1] == RAW;
              if (r0) Ev[h] = nib_bytes(uint32_t(rawv.f[0][i] >> (32 * h)));
              else Ev[h] = fieldv(0, h);
              if (r1) Mv[h] = tri_bytes(uint32_t(rawv.f[1][i] >> (24 * h)));
              else Mv[h] = fieldv(1, h);
            }
#pragma unroll
            for (int x = 0; x < 4; x++) {
              const uint32_t e4 = uint32_t(Ev[x >> 1] >> (32 * (x & 1)));
              const uint32_t m3 = uint32_t(Mv[x >> 1] >> (32 * (x & 1)));
              const uint32_t sg = uint32_t(rawv.plane[i] >> (4 * x)) & 15;
              // sign bits 0..3 to bits 7, 15, 23, 31
              o[x] = (e4 << 3) | m3 | (((sg * 0x204081u) << 7) & 0x80808080u);
            }
          }
          return o;
        };
        // Every lane stores one vector per iteration -- lanes without a
        // whole aligned vector store into the scratch sink -- so each round
        // issues the same stores and the compiler's waits for older loads
        // never have to drain them.
        bool partial = false;
#pragma unroll
        for (int i = 0; i < NVL; i++) {
          uint32_t ev;
          bool valid;
          const u32x4 o = vec(i, ev, valid);
          const bool whole = valid && ev + VE <= n && oaligned;
          stg16s(whole ? dst + uint64_t(ev) * ES : sink, o);
          partial |= valid && !whole;
          __builtin_amdgcn_sched_barrier(0);   // one vector at a time: fewer registers live
        }
        if (__ballot(partial)) {  // the last vectors of a tensor, or an unaligned output
#pragma unroll
          for (int i = 0; i < NVL; i++) {
            uint32_t ev;
            bool valid;
            const u32x4 o = vec(i, ev, valid);
            if (valid && !(ev + VE <= n && oaligned)) {
              uint8_t *op = dst + uint64_t(ev) * ES;
              const uint32_t cnt_b = (ev + VE <= n ? VE : n - ev) * ES;
              for (uint32_t b = 0; b < cnt_b; b++) stg1(op + b, o[b >> 2] >> ((b & 3) * 8));
            }
          }
        }
        wave_lds_sync();
      };
      // the first pair is peeled so that the loop is entered with the memory
      // operations of a whole round in flight, as on every later pass
      round(0, rawA, rawB);
      round(1, rawB, rawA);
      for (int r = 2; r < NR; r += 2) {
        round(r, rawA, rawB);
        round(r + 1, rawB, rawA);
      }
    }
    // each coded stream's segment lengths must add up to its payload
    if (coded && ln % SPW == 0 && wv == 0 && paybytes != 4 * ((seg_carry + 31) / 32)) bad = 1;
  };
  bool anyraw = false;
#pragma unroll
  for (int p = 0; p < NC; p++) anyraw |= sh.mode[p] == RAW;
  using I16 = std::integral_constant<int, 16>;
  using I32 = std::integral_constant<int, 32>;
  using I64 = std::integral_constant<int, 64>;
  using T = std::true_type;
  using F = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  using I12 = std::integral_constant<int, 12>;
  using I14 = std::integral_constant<int, 14>;
  // the same layouts with the first stream tANS-coded or not
  auto dispatch = [&](auto tc) {
    if (ncc == NC) {
      if constexpr (NC == 1) path(I64{}, F{}, T{}, I0{}, I0{}, tc);
      else if constexpr (NC == 2) path(I32{}, F{}, T{}, I0{}, I0{}, tc);
      else path(I16{}, F{}, T{}, I0{}, I0{}, tc);
    } else if constexpr (NC == 1) {
      if (anyraw) path(I64{}, T{}, F{}, I0{}, I0{}, tc); else path(I64{}, F{}, F{}, I0{}, I0{}, tc);
    } else if constexpr (NC == 2) {
      // usual FP8 weights: E4 coded, M3 raw
      if (ncc == 1 && rawm == 2) path(I64{}, T{}, F{}, I2{}, I0{}, tc);
      else if (anyraw) path(I64{}, T{}, F{}, I0{}, I0{}, tc);
      else path(I64{}, F{}, F{}, I0{}, I0{}, tc);
    } else {
      // usual FP32 weights: exponent coded, the three fraction bytes raw, or
      // the low two constant (values that are rounded BF16).  Any other mix
      // takes 16 lanes per stream, whatever ncc is: few vectors per lane keep
      // the registers of this rare case small.
      if (ncc == 1 && rawm == 14) path(I64{}, T{}, F{}, I14{}, I0{}, tc);
      else if (ncc == 1 && rawm == 2 && constm == 12) path(I64{}, T{}, F{}, I2{}, I12{}, tc);
      else if (anyraw) path(I16{}, T{}, F{}, I0{}, I0{}, tc);
      else path(I16{}, F{}, F{}, I0{}, I0{}, tc);
    }
  };
  if (sh.mode[0] == TANS) dispatch(T{});
  else dispatch(F{});
  if (bad) atomicOr(&a.ctl[0], kErrCorrupt);
}

__global__ void k_check(CheckArgs a) {
  const int tid = threadIdx.x;
  __shared__ int bad;
  if (tid == 0) bad = 0;
  __syncthreads();
  // this kernel runs first and owns the error word (ctl[0]) and the
  // container's group flag (ctl[1]): it stores, the decode reads and ORs
  if (a.in_bytes < a.hdr_bytes + 8ull * (a.n_chunks + 1)) {
    if (tid == 0) {
      a.ctl[0] = kErrCorrupt;
      a.ctl[1] = 0;
    }
    return;
  }
  for (uint32_t i = tid; i < a.hdr_bytes; i += blockDim.x) {
    if (i == 7 || (i >= 32 && i < 40) || (i >= 56 && i < 64)) continue;
    if (a.in[i] != a.hdr[i]) atomicOr(&bad, 1);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t err = bad ? kErrCorrupt : 0;
    const uint8_t flags = a.in[7];
    const uint64_t hash = *reinterpret_cast<const uint64_t *>(a.in + 32);
    const uint64_t total = *reinterpret_cast<const uint64_t *>(a.in + 56);
    if (flags > 1) err |= kErrCorrupt;
    if (flags == 1 && (a.K == 0 || hash != a.hash)) err |= kErrTableset;
    if (flags == 0 && hash != 0) err |= kErrCorrupt;
    if (total > a.in_bytes || (total & 15) || total < 16) err |= kErrCorrupt;
    else if (*reinterpret_cast<const uint64_t *>(a.in + a.off_dir + 8ull * a.n_chunks) != total - 16)
      err |= kErrCorrupt;
    a.ctl[0] = err;
    a.ctl[1] = flags == 1 ? 1u : 0u;
  }
}

hipError_t launch_check(const CheckArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL(k_check, dim3(1), dim3(256), 0, s, e0, e1, 0, a);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const DecArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.L.n_chunks == 0) return hipSuccess;
  const dim3 grid(a.L.n_chunks), block(DEC_NT);
  if (dtype == BF16) hipExtLaunchKernelGGL(k_decode<BF16>, grid, block, 0, s, e0, e1, 0, a);
  else if (dtype == FP32) hipExtLaunchKernelGGL(k_decode<FP32>, grid, block, 0, s, e0, e1, 0, a);
  else if (dtype == FP8) hipExtLaunchKernelGGL(k_decode<FP8>, grid, block, 0, s, e0, e1, 0, a);
  else hipExtLaunchKernelGGL(k_decode<FP4X2>, grid, block, 0, s, e0, e1, 0, a);
  return hipGetLastError();
}

}  // namespace zn
