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
constexpr int STWW = 10;       // staging words per lane: a strip and up to 5 symbols more
constexpr int RING = 32;       // words of a lane's payload window in LDS: two 64-byte sectors
// Staging and ring are lane-interleaved (word w of thread t at w * DEC_NT + t),
// so lanes that touch different words of their own areas still hit
// different LDS banks.

template <int DT>
struct DecShared {
  static constexpr int NC = ncoded(DT);
  uint32_t lut[NC][kLutSize];
  union {
    uint16_t t1[kLutSize];
    uint32_t stage[STWW * DEC_NT];
  } u;
  uint32_t ring[RING * DEC_NT];
  uint8_t len[NC][256];
  LutShared ls;
  int mode[NC], aux[NC];
  unsigned long long pay_off[NC], seg_off[NC];
  uint32_t pay[NC];
  uint32_t wtot[DEC_NT / 64][NC];   // [wave][coded stream index]
  int bad;
};

// Staged words w and w + 1 of thread t.
__device__ __forceinline__ uint64_t stg_pair(const uint32_t *stage, int w, int t) {
  return stage[w * DEC_NT + t] | (uint64_t(stage[(w + 1) * DEC_NT + t]) << 32);
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
      const uint32_t t = (w & 0x007F007Fu) | ((w >> 1) & ~0x007F007Fu);
      o[2 * h + x] = ((w << 8) & 0x80008000u) | (t & ~0x80008000u);
    }
  }
  return o;
}

template <int DT>
__global__ __launch_bounds__(DEC_NT) void k_decode(DecArgs a) {
  constexpr int NC = ncoded(DT), ES = esize(DT), S = segsyms(DT);
  constexpr int VE = 16 / ES;            // elements per 16-byte vector
  __shared__ DecShared<DT> sh;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  if (a.ctl[0]) return;  // the header check failed

  const uint32_t c = blockIdx.x;
  const int t = find_tensor(a.L, c);
  const uint64_t e0 = uint64_t(c - a.L.t_chunk0[t]) * a.L.chunk_elems;
  const uint64_t rem = a.L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < a.L.chunk_elems ? rem : a.L.chunk_elems);
  const int nseg = int((n + S - 1) / S);
  uint8_t *dst = a.out_ptrs[t] + e0 * ES;
  const bool oaligned = (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  const uint8_t *in = a.in;
  uint8_t *const sink = reinterpret_cast<uint8_t *>(a.ctl) + kSinkOff;
  const uint8_t *rawp = in + a.L.t_raw[t] + (DT == BF16 ? e0 : DT == FP8 ? e0 / 8 : 0);

  // ------------------------------------------------- 1. walk the record
  if (tid == 0) {
    int bad = 0;
    const uint64_t *dir = reinterpret_cast<const uint64_t *>(in + a.L.off_dir);
    const uint64_t r0 = dir[c], r1 = dir[c + 1];
    if (r0 < a.L.off_records || r1 < r0 || r1 + 16 > a.in_bytes || (r0 & 15)) bad = 1;
    uint64_t pos = r0;
    for (int p = 0; p < NC && !bad; p++) {
      const int k = kbits(DT, p), A = 1 << k;
      if (pos + 16 > r1) { bad = 1; break; }
      const uint32_t h0 = *reinterpret_cast<const uint32_t *>(in + pos);
      const uint32_t pay = *reinterpret_cast<const uint32_t *>(in + pos + 4);
      const int mode = h0 & 0xFF, aux = (h0 >> 8) & 0xFF, ns = h0 >> 16;
      if (mode > GROUP || ns != nseg) { bad = 1; break; }
      const uint64_t head = head_bytes_of(mode, k, nseg);
      if (pos + head + align16(pay) > r1) { bad = 1; break; }
      if (mode == CONST && (aux >= A || pay != 0)) bad = 1;
      if (mode == RAW && (aux != 0 || pay != (uint64_t(n) * k + 7) / 8)) bad = 1;
      if (mode == HUFF && (aux != 0 || pay == 0 || (pay & 3))) bad = 1;
      if (mode == GROUP && (p != 0 || aux >= a.K || pay == 0 || (pay & 3))) bad = 1;
      sh.mode[p] = mode;
      sh.aux[p] = aux;
      sh.pay[p] = pay;
      sh.pay_off[p] = pos + head;
      sh.seg_off[p] = pos + 8 + (mode == HUFF ? A / 2 : 0);
      pos += head + align16(pay);
    }
    if (!bad && pos != r1) bad = 1;
    sh.bad = bad;
  }
  __syncthreads();
  if (sh.bad) {
    if (tid == 0) atomicOr(&a.ctl[0], kErrCorrupt);
    return;
  }

  // ---------------------------------------------------------- 2. tables
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k, mode = sh.mode[p];
    if (mode == HUFF) {
      const uint8_t *nib = in + sh.seg_off[p] - A / 2;
      if (tid < A) sh.len[p][tid] = (ldg1(nib + (tid >> 1)) >> ((tid & 1) * 4)) & 15;
      __syncthreads();
      if (!build_lut<DEC_NT>(sh.len[p], A, sh.lut[p], sh.u.t1, sh.ls)) {
        if (tid == 0) atomicOr(&a.ctl[0], kErrCorrupt);
        return;
      }
    } else if (mode == GROUP) {
      const uint32_t *gl = a.group_lut + size_t(sh.aux[p]) * kLutSize;
      for (int i = tid; i < kLutSize; i += DEC_NT) sh.lut[p][i] = ldg4(gl + i);
      if (tid < A) sh.len[p][tid] = ldg1(a.group_len + sh.aux[p] * 256 + tid);
    }
  }
  __syncthreads();

  // ------------------------------------------------ 3. lanes and rounds
  // Lanes decode only the Huffman- or group-coded streams; raw and constant
  // streams need no decoding and the merge reads them straight from the
  // record.  With ncc coded streams, SPW = 64, 32 or 16 lanes of each wave
  // take one coded stream each (a template per SPW; the branch below is
  // uniform per workgroup).
  int ncc = 0, cs[NC], cidx[NC];
#pragma unroll
  for (int p = 0; p < NC; p++) {
    cidx[p] = -1;
    if (sh.mode[p] == HUFF || sh.mode[p] == GROUP) { cs[ncc] = p; cidx[p] = ncc; ncc++; }
  }
  // Fields of the raw streams for one 16-byte output vector of VE elements
  // starting at element ev (< n): k = 8 gives VE bytes, k = 4 VE nibbles,
  // k = 3 a 3*VE-bit run.  Every read stays inside the stream's payload, or
  // at most 4 bytes past it where the record or the container tail follows
  // (the record walk checked that the container holds them).
  auto raw_field = [&](int p, uint32_t ev) -> uint64_t {
    const uint8_t *pay = in + sh.pay_off[p];
    const int k = kbits(DT, p);
    if (k == 8) {
      if constexpr (VE == 8) { const u32x2 x = ldg8(pay + ev); return x[0] | (uint64_t(x[1]) << 32); }
      else if constexpr (VE == 4) return ldg4(pay + ev);
      else return 0;
    }
    if (k == 4) { const u32x2 x = ldg8(pay + ev / 2); return x[0] | (uint64_t(x[1]) << 32); }
    const uint32_t b = ev * 3, w0 = b >> 5;   // ev is a multiple of 16: b & 31 is 0 or 16
    const uint64_t x = ldg4(pay + 4 * w0) | (uint64_t(ldg4(pay + 4 * w0 + 4)) << 32);
    return x >> (b & 31);
  };
  // a constant stream's byte in every byte lane
  auto cfield = [&](int p) -> uint64_t { return 0x0101010101010101ull * uint64_t(sh.aux[p]); };

  int bad = 0;
  auto path = [&](auto spw_c, auto rawf_c) {
    constexpr int SPW = decltype(spw_c)::value;   // lanes per coded stream per wave
    constexpr bool RAWF = decltype(rawf_c)::value; // some stream is stored raw
    constexpr int GS = 4 * SPW;                   // segments per coded stream per group
    constexpr int VPS = RND * ES / 16;            // output vectors per strip
    constexpr int NVL = SPW * VPS / 64;           // output vectors per lane per round
    // Lane (wave wv, lane ln) decodes coded stream ci = ln / SPW, segment slot
    // wv*SPW + ln%SPW.  Round r decodes strip r*nseg + j of every segment j,
    // so one round of a wave covers SPW consecutive strips: a contiguous
    // block of the output.
    const int ci = ln / SPW, slot = wv * SPW + ln % SPW;
    const bool coded = ci < ncc;
    const int p = coded ? cs[ci] : 0;
    const uint8_t *pay = in + sh.pay_off[p];
    const uint32_t paybytes = sh.pay[p];
    const uint32_t ngroups = (paybytes + 15) / 16;
    const uint32_t *lut = sh.lut[p];
    uint32_t *sp = sh.u.stage + tid;    // staged word w of this lane: sp[w * DEC_NT]
    uint32_t *rp = sh.ring + tid;       // ring word w of this lane: rp[w * DEC_NT]
    const int t0 = wv * 64;             // first thread of this wave
    uint32_t seg_carry = 0;
    const uint32_t nstrips = (n + RND - 1) / RND;
    const int G = (nseg + GS - 1) / GS;
    for (int g = 0; g < G; g++) {
      const int sj = g * GS + slot;
      const bool live = sj < nseg;
      // start bit of the segment: scan of the stored segment bit lengths
      uint32_t sbits = 0;
      if (coded && live) sbits = ldg2(in + sh.seg_off[p] + 2 * sj);
      const uint32_t incl = wave_incl_scan(sbits);
      const int first = ci * SPW;
      const uint32_t wbase = first > 0 ? __shfl(incl, first - 1, 64) : 0;
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

      // Bit reader: a 64-bit window (LSB-first) refilled one word at a time
      // from the lane's ring of payload words in LDS.  The ring holds two
      // 64-byte sectors of the payload, aligned in memory so that every
      // sector is one HBM burst read once; a sector is loaded one round
      // before it can be needed.  Word positions count from the aligned base.
      uint64_t buf = 0;
      int nb = 0;
      const uintptr_t pa = reinterpret_cast<uintptr_t>(pay);
      const uint8_t *pay64 = pay - (pa & 63);       // inside the container: pay is past the header
      const uint32_t adj = uint32_t(pa & 63) / 4;   // payload word 0 is window word adj
      const uint32_t glast = adj / 4 + ngroups - 1; // last 16-byte group holding payload
      uint32_t wpos = 0, nsec = 0, pre = 0;         // next word to read, next sector to fetch
      u32x4 ps0 = {0, 0, 0, 0}, ps1 = ps0, ps2 = ps0, ps3 = ps0;
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
        const u32x4 a0 = grp(4 * s0), a1 = grp(4 * s0 + 1), a2 = grp(4 * s0 + 2), a3 = grp(4 * s0 + 3);
        const u32x4 a4 = grp(4 * s0 + 4), a5 = grp(4 * s0 + 5), a6 = grp(4 * s0 + 6), a7 = grp(4 * s0 + 7);
        put_sector(s0, a0, a1, a2, a3);
        put_sector(s0 + 1, a4, a5, a6, a7);
        nsec = s0 + 2;
        buf = rp[(w0 & (RING - 1)) * DEC_NT] | (uint64_t(rp[((w0 + 1) & (RING - 1)) * DEC_NT]) << 32);
        wpos = w0 + 2;
        buf >>= (b0 & 31);
        nb = 64 - int(b0 & 31);
      }
      int ov = 0;         // symbols of the next strip decoded early (staged words 8, 9)
      // Raw bits and raw-stream fields merged by this lane in round r: the
      // same loads every round (an empty vector reads element 0 and is
      // ignored), so no wait has to drain the stores in flight.  A partial
      // last vector stays inside the always-raw plane, whose size is padded
      // to 16 bytes: BF16 vectors start at multiples of 8 bytes, FP8 sign
      // words at multiples of 2.
      using FT = std::conditional_t<ES == 4, uint32_t, uint64_t>;  // VE raw-stream fields
      struct RawIn { uint64_t plane[NVL]; FT f[NC][NVL]; };
      auto load_raw = [&](int r, RawIn &rv) {
#pragma unroll
        for (int i = 0; i < NVL; i++) {
          const int v = ln + 64 * i, sl = v / VPS, part = v % VPS;
          const int sjv = g * GS + wv * SPW + sl;
          const uint32_t ev0 = (uint32_t(r) * nseg + sjv) * RND + part * VE;
          const uint32_t ev = sjv < nseg && ev0 < n ? ev0 : 0;
          if constexpr (DT == BF16) {
            const u32x2 x = ldg8s(rawp + ev);
            rv.plane[i] = x[0] | (uint64_t(x[1]) << 32);
          } else if constexpr (DT == FP8) {
            rv.plane[i] = ldg2(rawp + ev / 8);
          } else {
            rv.plane[i] = 0;
          }
          if constexpr (RAWF) {
#pragma unroll
            for (int q = 0; q < NC; q++) rv.f[q][i] = sh.mode[q] == RAW ? FT(raw_field(q, ev)) : FT(0);
          }
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
        load_raw(r + 1 < NR ? r + 1 : r, nxt);  // the last round reloads its own: same count
        const uint32_t q = uint32_t(r) * nseg + sj;   // this lane's strip
        const int lim = coded && live && q < nstrips ? int(min(uint32_t(RND), n - q * RND)) : 0;
        const bool last = live && q < nstrips && q + nseg >= nstrips;
        // the sector fetched last round enters the ring
        if (pend) {
          put_sector(nsec, ps0, ps1, ps2, ps3);
          nsec++;
          pend = false;
        }
        if (lim > 0) {
          // Symbols are staged four to a word.  cur holds the bytes of the
          // word being filled; each lookup writes that word and the next
          // (aligned stores; the next word holds what spilled over) and
          // moves on when the word is complete -- no branch per lookup.
          // The window is refilled, also without branches, with 32 bits
          // whenever fewer than 32 remain: enough for the two lookups of an
          // iteration (at most 22 bits).
          uint32_t cur = 0;
          uint32_t *wp = sp;        // the word being filled
          if (ov) {  // symbols of this strip decoded last round: words 8, 9 -> 0, 1
            const uint32_t c8 = sp[8 * DEC_NT], c9 = sp[9 * DEC_NT];
            sp[0] = c8;
            sp[DEC_NT] = c9;
            cur = ov >= 4 ? c9 : c8;
            wp = ov >= 4 ? sp + DEC_NT : sp;
          }
          int pos = ov;             // symbols of this strip decoded so far
          uint32_t na = ov & 3;     // bytes in cur
          pre = rp[(wpos & (RING - 1)) * DEC_NT];
          auto emit = [&](uint32_t e) {
            const uint64_t tt = uint64_t(e & 0xFFFFFF) << (8 * na);
            const uint32_t lo = cur | uint32_t(tt), hi = uint32_t(tt >> 32);
            wp[0] = lo;
            wp[DEC_NT] = hi;
            const uint32_t m = e >> 28;
            pos += int(m);
            na += m;
            const bool full = na >= 4;
            cur = full ? hi : lo;
            wp += full ? DEC_NT : 0;
            na &= 3;
          };
          while (pos < lim) {
            const bool need = nb < 32;
            buf |= uint64_t(need ? pre : 0u) << nb;
            nb += need ? 32 : 0;
            wpos += need ? 1u : 0u;
            pre = rp[(wpos & (RING - 1)) * DEC_NT];
            uint32_t e = lut[buf & (kLutSize - 1)];
            emit(e);
            uint32_t bl = (e >> 24) & 15;
            buf >>= bl;
            nb -= int(bl);
            e = lut[buf & (kLutSize - 1)];
            emit(e);
            bl = (e >> 24) & 15;
            buf >>= bl;
            nb -= int(bl);
          }
          ov = pos - lim;   // at most 5: the loop stops 2 lookups of 3 symbols past lim - 1
          if (last) {
            // exact end: the segment must use exactly its stored bit length
            uint64_t bpos = uint64_t(wpos - adj) * 32 - uint32_t(nb);
            for (int x = 0; x < ov; x++) {
              const int bb = lim + x;
              bpos -= sh.len[p][(sp[(bb >> 2) * DEC_NT] >> (8 * (bb & 3))) & 0xFF];
            }
            if (bpos != uint64_t(b0) + sbits) bad = 1;
            ov = 0;
          } else if (((wpos + 11) >> 4) >= nsec) {
            // lim == RND here.  The next round reads at most 32 lookups (352
            // bits) with at least 10 bits left in the window, so words
            // [wpos, wpos + 12): at most one sector past those in the ring,
            // whose slot held a sector before wpos's.
            ps0 = grp(4 * nsec);
            ps1 = grp(4 * nsec + 1);
            ps2 = grp(4 * nsec + 2);
            ps3 = grp(4 * nsec + 3);
            pend = true;
          }
        }
        wave_lds_sync();
        // merge and store: vector v of this wave covers VE elements of slot v / VPS
#pragma unroll
        for (int i = 0; i < NVL; i++) {
          const int v = ln + 64 * i, sl = v / VPS, part = v % VPS;
          const int sjv = g * GS + wv * SPW + sl;
          const uint32_t qv = uint32_t(r) * nseg + sjv;
          const uint32_t ev = qv * RND + part * VE;
          const bool valid = sjv < nseg && ev < n;
          // staged bytes of coded stream pp for this vector (VE bytes)
          auto staged = [&](int pp, int h) -> uint64_t {
            const int th = t0 + cidx[pp] * SPW + sl;
            if constexpr (ES == 2) return stg_pair(sh.u.stage, 2 * part, th);
            else if constexpr (ES == 4) return sh.u.stage[part * DEC_NT + th];
            else return stg_pair(sh.u.stage, 4 * part + 2 * h, th);
          };
          auto fieldv = [&](int pp, int h) -> uint64_t {   // h: 8-byte half (FP8)
            const int md = sh.mode[pp];
            if (md == CONST) return cfield(pp);
            if (md != RAW || !RAWF) return staged(pp, h);
            return rawv.f[pp][i];
          };
          u32x4 o;
          if constexpr (DT == BF16) {
            o = merge_bf16(fieldv(0, 0), rawv.plane[i]);
          } else if constexpr (DT == FP32) {
            uint32_t P[4];
#pragma unroll
            for (int pp = 0; pp < 4; pp++) P[pp] = uint32_t(fieldv(pp, 0));
#pragma unroll
            for (int x = 0; x < 4; x++) {
              const uint32_t p0 = (P[0] >> (8 * x)) & 0xFF, p1 = (P[1] >> (8 * x)) & 0xFF;
              const uint32_t p2 = (P[2] >> (8 * x)) & 0xFF, p3 = (P[3] >> (8 * x)) & 0xFF;
              o[x] = ((p1 & 0x80) << 24) | (p0 << 23) | ((p1 & 0x7F) << 16) | (p2 << 8) | p3;
            }
          } else {
            // E4 and M3 of the 16 elements as bytes, from whichever source
            uint64_t Ev[2], Mv[2];
            const int m0 = sh.mode[0], m1 = sh.mode[1];
#pragma unroll
            for (int h = 0; h < 2; h++) {
              if (m0 == RAW) {
                const uint64_t x = rawv.f[0][i] >> (32 * h);   // 8 nibbles
                uint64_t y = 0;
#pragma unroll
                for (int j = 0; j < 8; j++) y |= ((x >> (4 * j)) & 15) << (8 * j);
                Ev[h] = y;
              } else {
                Ev[h] = fieldv(0, h);
              }
              if (m1 == RAW) {
                const uint64_t x = rawv.f[1][i] >> (24 * h);   // 8 values of 3 bits
                uint64_t y = 0;
#pragma unroll
                for (int j = 0; j < 8; j++) y |= ((x >> (3 * j)) & 7) << (8 * j);
                Mv[h] = y;
              } else {
                Mv[h] = fieldv(1, h);
              }
            }
#pragma unroll
            for (int x = 0; x < 4; x++) {
              const uint32_t e4 = uint32_t(Ev[x >> 1] >> (32 * (x & 1)));
              const uint32_t m3 = uint32_t(Mv[x >> 1] >> (32 * (x & 1)));
              const uint32_t sg = uint32_t(rawv.plane[i] >> (4 * x)) & 15;
              const uint32_t sb = ((sg & 1) << 7) | ((sg & 2) << 14) | ((sg & 4) << 21) | ((sg & 8) << 28);
              o[x] = (e4 << 3) | m3 | sb;
            }
          }
          // Every lane stores one vector per iteration -- lanes without a
          // whole aligned vector store into the scratch sink -- so each round
          // issues the same stores and the compiler's waits for older loads
          // never have to drain them.
          uint8_t *op = dst + uint64_t(ev) * ES;
          const bool whole = valid && ev + VE <= n && oaligned;
          stg16(whole ? op : sink, o);
          if (valid && !whole) {  // a partial last vector or an unaligned output
            const uint32_t cnt_b = (ev + VE <= n ? VE : n - ev) * ES;
            for (uint32_t b = 0; b < cnt_b; b++) stg1(op + b, o[b >> 2] >> ((b & 3) * 8));
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
  if (ncc <= 1) {
    if (anyraw) path(I64{}, T{}); else path(I64{}, F{});
  } else if constexpr (NC >= 2) {
    if (ncc == 2) {
      if (anyraw) path(I32{}, T{}); else path(I32{}, F{});
    } else if constexpr (NC == 4) {
      if (anyraw) path(I16{}, T{}); else path(I16{}, F{});
    }
  }
  if (bad) atomicOr(&a.ctl[0], kErrCorrupt);
}

__global__ void k_check(CheckArgs a) {
  const int tid = threadIdx.x;
  __shared__ int bad;
  if (tid == 0) bad = 0;
  __syncthreads();
  // this kernel runs first and owns the error word: it stores, the decode ORs
  if (a.in_bytes < a.hdr_bytes + 8ull * (a.n_chunks + 1)) {
    if (tid == 0) a.ctl[0] = kErrCorrupt;
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
  }
}

hipError_t launch_check(const CheckArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_check, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const DecArgs &a, hipStream_t s) {
  if (a.L.n_chunks == 0) return hipSuccess;
  const dim3 grid(a.L.n_chunks), block(DEC_NT);
  if (dtype == BF16) hipLaunchKernelGGL(k_decode<BF16>, grid, block, 0, s, a);
  else if (dtype == FP32) hipLaunchKernelGGL(k_decode<FP32>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_decode<FP8>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace zn
