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
#include "zn_internal.h"

namespace zn {

constexpr int DEC_NT = 256;
constexpr int RND = 32;        // symbols per lane per round
constexpr int STW = RND + 8;   // staging bytes per lane (overflow slack, 8-byte multiple)

template <int DT>
struct DecShared {
  static constexpr int NC = ncoded(DT);
  uint32_t lut[NC][kLutSize];
  union {
    uint16_t t1[kLutSize];
    uint8_t stage[DEC_NT * STW];
  } u;
  uint8_t len[NC][256];
  LutShared ls;
  int mode[NC], aux[NC];
  unsigned long long pay_off[NC], seg_off[NC];
  uint32_t pay[NC];
  uint32_t wtot[DEC_NT / 64];
  int bad;
};

template <int DT>
__device__ __forceinline__ uint32_t merge_elem(const uint32_t *sym, uint32_t raw) {
  if constexpr (DT == BF16) return ((raw & 0x80) << 8) | (sym[0] << 7) | (raw & 0x7F);
  if constexpr (DT == FP32)
    return ((sym[1] & 0x80) << 24) | (sym[0] << 23) | ((sym[1] & 0x7F) << 16) | (sym[2] << 8) | sym[3];
  return ((raw & 1) << 7) | (sym[0] << 3) | sym[1];
}

template <int DT>
__global__ __launch_bounds__(DEC_NT) void k_decode(DecArgs a) {
  constexpr int NC = ncoded(DT), ES = esize(DT), S = segsyms(DT);
  constexpr int LPS = DEC_NT / NC;       // lanes per stream
  constexpr int VE = 16 / ES;            // elements per 16-byte vector
  constexpr int VPS = RND * ES / 16;     // vectors per segment per round
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
      if (tid < A) sh.len[p][tid] = (nib[tid >> 1] >> ((tid & 1) * 4)) & 15;
      __syncthreads();
      if (!build_lut<DEC_NT>(sh.len[p], A, sh.lut[p], sh.u.t1, sh.ls)) {
        if (tid == 0) atomicOr(&a.ctl[0], kErrCorrupt);
        return;
      }
    } else if (mode == GROUP) {
      const uint32_t *gl = a.group_lut + size_t(sh.aux[p]) * kLutSize;
      for (int i = tid; i < kLutSize; i += DEC_NT) sh.lut[p][i] = gl[i];
      if (tid < A) sh.len[p][tid] = a.group_len[sh.aux[p] * 256 + tid];
    }
  }
  __syncthreads();

  // ------------------------------------------------ 3. lanes and rounds
  const int p = tid / LPS, j = tid % LPS, k = kbits(DT, p);
  const int mode = sh.mode[p];
  const bool coded = mode == HUFF || mode == GROUP;
  const uint4 *P4 = reinterpret_cast<const uint4 *>(in + sh.pay_off[p]);
  const uint32_t ngroups = (sh.pay[p] + 15) / 16;
  const uint32_t *lut = sh.lut[p];
  uint8_t *st = sh.u.stage + tid * STW;
  uint32_t seg_carry = 0;  // bits of the stream's segments in earlier groups
  int bad = 0;
  const int G = (nseg + LPS - 1) / LPS;
  for (int g = 0; g < G; g++) {
    const int sj = g * LPS + j;
    const bool live = sj < nseg;
    const int slen = live ? int(min(uint32_t(S), n - uint32_t(sj) * S)) : 0;
    // start bit of this lane's segment: scan of the stored segment lengths
    uint32_t sbits = 0;
    if (coded && live) sbits = reinterpret_cast<const uint16_t *>(in + sh.seg_off[p])[sj];
    const uint32_t incl = wave_incl_scan(sbits);
    if (ln == 63) sh.wtot[wv] = incl;
    __syncthreads();
    uint32_t before = 0, gtot = 0;
    for (int q = 0; q < DEC_NT / 64; q++) {
      if (q * 64 / LPS != p) continue;  // waves of this lane's stream
      before += q < wv ? sh.wtot[q] : 0;
      gtot += sh.wtot[q];
    }
    const uint32_t b0 = seg_carry + before + incl - sbits;
    seg_carry += gtot;
    __syncthreads();

    // bit reader state (LSB-first): 64-bit window, 16-byte prefetch queue
    unsigned long long buf = 0;
    int nb = 0;
    uint4 q0 = make_uint4(0, 0, 0, 0), q1 = q0;
    uint32_t gnext = 0, wtaken = 0;
    int qi = 0;
    auto grp = [&](uint32_t gi) { return P4[gi < ngroups ? gi : ngroups - 1]; };
    auto take = [&]() -> uint32_t {
      const uint32_t x = qi == 0 ? q0.x : qi == 1 ? q0.y : qi == 2 ? q0.z : q0.w;
      wtaken++;
      if (++qi == 4) {
        q0 = q1;
        q1 = grp(gnext++);
        qi = 0;
      }
      return x;
    };
    if (coded && live) {
      const uint32_t w0 = b0 >> 5;
      gnext = (w0 >> 2);
      q0 = grp(gnext++);
      q1 = grp(gnext++);
      qi = int(w0 & 3);
      wtaken = w0;
      buf = take();
      buf |= (unsigned long long)take() << 32;
      buf >>= (b0 & 31);
      nb = 64 - int(b0 & 31);
    }
    int ov = 0;          // symbols decoded past the previous round's end
    uint32_t carry = 0;  // those symbols
    const int rounds = S / RND;
    for (int r = 0; r < rounds; r++) {
      const int base = r * RND;
      const int lim = slen - base < RND ? (slen - base > 0 ? slen - base : 0) : RND;
      // prefetch of the raw bits this thread merges after the round
      constexpr int NVT = (LPS * VPS + DEC_NT - 1) / DEC_NT;
      unsigned long long rawv[NVT];
      const int nsg = nseg - g * LPS < LPS ? nseg - g * LPS : LPS;
#pragma unroll
      for (int i = 0; i < NVT; i++) {
        rawv[i] = 0;
        const int v = tid + i * DEC_NT;
        const int sjv = g * LPS + v / VPS;
        const uint32_t ev = uint32_t(sjv) * S + base + (v % VPS) * VE;
        if (v / VPS < nsg && ev < n) {
          if constexpr (DT == BF16) {
            const uint8_t *rp = in + a.L.t_raw[t] + e0 + ev;
            if (ev + VE <= n) rawv[i] = *reinterpret_cast<const unsigned long long *>(rp);
            else for (uint32_t q = 0; ev + q < n; q++) rawv[i] |= (unsigned long long)rp[q] << (8 * q);
          } else if constexpr (DT == FP8) {
            const uint8_t *rp = in + a.L.t_raw[t] + (e0 + ev) / 8;
            rawv[i] = rp[0] | (ev + 8 < n ? uint32_t(rp[1]) << 8 : 0u);
          }
        }
      }
      if (lim > 0) {
        if (coded) {
          int cnt = ov;
          if (ov > 0) st[0] = uint8_t(carry);
          if (ov > 1) st[1] = uint8_t(carry >> 8);
          uint32_t e = 0;
          while (cnt < lim) {
            if (nb < 32) {
              buf |= (unsigned long long)take() << nb;
              nb += 32;
            }
            e = lut[buf & (kLutSize - 1)];
            st[cnt] = uint8_t(e);
            st[cnt + 1] = uint8_t(e >> 8);
            st[cnt + 2] = uint8_t(e >> 16);
            cnt += int(e >> 28);
            const int bl = int((e >> 24) & 15);
            buf >>= bl;
            nb -= bl;
          }
          ov = cnt - lim;
          carry = ov > 0 ? (uint32_t(st[lim]) | (uint32_t(st[lim + 1]) << 8)) : 0;
          if (base + lim == slen) {
            // exact end: the segment must use exactly its stored bit length
            uint64_t pos = uint64_t(wtaken) * 32 - uint32_t(nb);
            for (int q = 0; q < ov; q++) pos -= sh.len[p][(carry >> (8 * q)) & 0xFF];
            if (pos != uint64_t(b0) + sbits) bad = 1;
          }
        } else if (mode == RAW) {
          // k-bit values, value bit 0 first; a round spans whole words
          const uint64_t i0 = uint64_t(sj) * S + base;
          const uint32_t *pw = reinterpret_cast<const uint32_t *>(in + sh.pay_off[p]);
          const uint64_t wbase = i0 * k / 32;
          const uint32_t maxw = (sh.pay[p] + 15) / 16 * 4;
          uint32_t wds[8];
#pragma unroll
          for (int q = 0; q < 8; q++)
            wds[q] = (q < k && wbase + q < maxw) ? pw[wbase + q] : 0u;
#pragma unroll
          for (int m = 0; m < RND; m++) {
            const int bit = m * k;
            const uint32_t lo = wds[bit >> 5] >> (bit & 31);
            const uint32_t hi = (bit & 31) + k > 32 ? wds[(bit >> 5) + 1] << (32 - (bit & 31)) : 0u;
            st[m] = uint8_t((lo | hi) & ((1u << k) - 1));
          }
        }
      }
      __syncthreads();
      // merge and store: vector v covers VE elements of segment v / VPS
#pragma unroll
      for (int i = 0; i < NVT; i++) {
        const int v = tid + i * DEC_NT;
        const int js = v / VPS, part = v % VPS;
        const uint32_t ev = uint32_t(g * LPS + js) * S + base + part * VE;
        if (js >= nsg || ev >= n) continue;
        uint32_t outw[4] = {0, 0, 0, 0};
        const int cnt_e = ev + VE <= n ? VE : int(n - ev);
        for (int q = 0; q < VE; q++) {
          uint32_t sym[4] = {0, 0, 0, 0};
#pragma unroll
          for (int pp = 0; pp < NC; pp++) {
            const int mp = sh.mode[pp];
            sym[pp] = mp == CONST ? uint32_t(sh.aux[pp])
                                  : sh.u.stage[(pp * LPS + js) * STW + part * VE + q];
          }
          uint32_t raw = 0;
          if constexpr (DT == BF16) raw = uint32_t(rawv[i] >> (8 * q)) & 0xFF;
          if constexpr (DT == FP8) raw = uint32_t(rawv[i] >> q) & 1;
          const uint32_t w = merge_elem<DT>(sym, raw);
          outw[(q * ES) >> 2] |= w << (((q * ES) & 3) * 8);
        }
        uint8_t *op = dst + uint64_t(ev) * ES;
        if (cnt_e == VE && oaligned) {
          *reinterpret_cast<uint4 *>(op) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
        } else {
          for (int b = 0; b < cnt_e * ES; b++) op[b] = uint8_t(outw[b >> 2] >> ((b & 3) * 8));
        }
      }
      __syncthreads();
    }
  }
  // the stream's segment lengths must add up to its payload
  if (coded && j == 0 && sh.pay[p] != 4 * ((seg_carry + 31) / 32)) bad = 1;
  if (bad) atomicOr(&a.ctl[0], kErrCorrupt);
}

__global__ void k_check(CheckArgs a) {
  const int tid = threadIdx.x;
  __shared__ int bad;
  if (tid == 0) bad = 0;
  __syncthreads();
  if (a.in_bytes < a.hdr_bytes + 8ull * (a.n_chunks + 1)) {
    if (tid == 0) atomicOr(a.ctl, kErrCorrupt);
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
    if (err) atomicOr(a.ctl, err);
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
