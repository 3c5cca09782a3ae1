// zn_encode.hip -- the compression pass for gfx950.
//
// One workgroup of 512 threads (8 wave64s) per chunk, in one launch:
//   1. read the chunk once with 16-byte loads, split every element into its
//      coded fields and its always-raw bits (THEORY-599 on ZipNN, per-field
//      compressibility, ZipNN Table II), store the raw bits straight to their
//      final place, and count each coded field in LDS histograms privatised
//      per lane column (the exponent histogram is very skewed: a handful of
//      bins take most hits, so lanes must not share counters);
//   2. per coded stream: constant / shared group code / own optimal code /
//      raw, by exact section size; the own code is built in LDS by
//      package-merge (THEORY-599, order-0 only; "NeuralZip: Reusable Setup
//      for Fast Lossless Compression", Abstract, for group codes);
//   3. the record size is known from the histogram alone, so the record's
//      offset comes from a decoupled look-back over the chunks that took
//      earlier tickets (chunks run in ticket order, so every predecessor is
//      resident or done);
//   4. re-read the chunk (it is still in L2 / Infinity Cache) and pack codes:
//      one wave per segment, a wave scan of bit counts, code words ORed into
//      an LDS tile, whole 32-bit words stored coalesced.
#include "zn_internal.h"

namespace zn {

constexpr int ENC_NT = 512;
constexpr unsigned long long FLAG_AGG = 1ull << 62, FLAG_INC = 2ull << 62;
constexpr unsigned long long VALUE_MASK = (1ull << 62) - 1;
constexpr int SPIN_LIMIT = 1 << 24;

template <int DT, int P>
__device__ __forceinline__ uint32_t field(uint32_t w) {
  if constexpr (DT == BF16) return (w >> 7) & 0xFF;
  if constexpr (DT == FP32) {
    if constexpr (P == 0) return (w >> 23) & 0xFF;
    if constexpr (P == 1) return ((w >> 24) & 0x80) | ((w >> 16) & 0x7F);
    if constexpr (P == 2) return (w >> 8) & 0xFF;
    return w & 0xFF;
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

template <int DT>
struct EncShared {
  static constexpr int NC = ncoded(DT);
  static constexpr int S = segsyms(DT);
  static constexpr int COLS = DT == FP32 ? 16 : 32;
  static constexpr int APRIV = DT == FP8 ? (16 + 8) : 256 * NC;   // total bins
  static constexpr int STAGE = (8 * S * kMaxLen + 31) / 32 + 4;   // words of one pack tile
  uint32_t hist[NC][256];
  uint32_t enc[NC][256];
  uint8_t len[NC][256];
  unsigned long long bits[NC];
  unsigned long long sec_off[NC + 1];
  int mode[NC], aux[NC];
  unsigned long long rsum[8];
  int icnt[8];
  uint32_t chunk;
  unsigned long long excl;
  int cnt[4][kMaxLen + 1];
  union {
    uint32_t priv[APRIV * COLS];
    struct {
      PMShared pm;
      uint64_t hw[256];
    } cb;
    struct {
      uint32_t stage[STAGE];
      uint32_t wtot[8];
    } pk;
  } u;
};

template <int DT>
__device__ __forceinline__ int priv_base(int p) {
  if constexpr (DT == FP8) return p == 0 ? 0 : 16;
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
  for (int w = 0; w < ENC_NT / 64; w++) t += sh.rsum[w];
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
  for (int w = 0; w < ENC_NT / 64; w++) t += sh.icnt[w];
  return t;
}

template <int DT>
__global__ __launch_bounds__(ENC_NT) void k_encode(EncArgs a) {
  constexpr int NC = ncoded(DT), ES = esize(DT), S = segsyms(DT);
  constexpr int VE = 16 / ES;          // elements per 16-byte vector
  constexpr int EPT = S / 64;          // elements per thread per pack tile (a wave = a segment)
  constexpr int NV = EPT / VE;         // vectors per thread per pack tile
  constexpr int COLS = EncShared<DT>::COLS;
  __shared__ EncShared<DT> sh;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;

  // ---------------------------------------------------------------- ticket
  if (tid == 0) sh.chunk = atomicAdd(&a.ctl[1], 1u);
  __syncthreads();
  const uint32_t c = sh.chunk;
  if (c >= a.L.n_chunks) return;
  const int t = find_tensor(a.L, c);
  const uint64_t e0 = uint64_t(c - a.L.t_chunk0[t]) * a.L.chunk_elems;
  const uint64_t rem = a.L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < a.L.chunk_elems ? rem : a.L.chunk_elems);
  const uint8_t *src = a.in_ptrs[t] + e0 * ES;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const uint32_t nvec = aligned ? n / VE : 0;
  uint8_t *rawp = a.out + a.L.t_raw[t];

  // ------------------------------------------- 1. split, raw planes, counts
  for (int i = tid; i < EncShared<DT>::APRIV * COLS; i += ENC_NT) sh.u.priv[i] = 0;
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
#pragma unroll
        for (int p = 0; p < NC; p++)
          atomicAdd(&sh.u.priv[(priv_base<DT>(p) + field_rt<DT>(w, p)) * COLS + col], 1u);
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
      }
    }
  }
  for (uint32_t i = nvec * VE + tid; i < n; i += ENC_NT) {  // ragged tail or unaligned input
    const uint32_t w = load_elem<DT>(src + uint64_t(i) * ES);
#pragma unroll
    for (int p = 0; p < NC; p++)
      atomicAdd(&sh.u.priv[(priv_base<DT>(p) + field_rt<DT>(w, p)) * COLS + col], 1u);
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
  __syncthreads();
  for (int i = tid; i < EncShared<DT>::APRIV; i += ENC_NT) {
    uint32_t s = 0;
    for (int j = 0; j < COLS; j++) s += sh.u.priv[i * COLS + ((j + i) & (COLS - 1))];
    int p = 0, sym = i;
    if constexpr (DT == FP8) { p = i >= 16; sym = i - (p ? 16 : 0); }
    else { p = i >> 8; sym = i & 255; }
    sh.hist[p][sym] = s;
  }
  __syncthreads();

  // --------------------------------------------- 2. mode and code per stream
  const int nseg = int((n + S - 1) / S);
  unsigned long long rec = 0;
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k;
    const uint32_t h = tid < A ? sh.hist[p][tid] : 0;
    const int d = block_count<DT>(sh, h != 0);
    int mode;
    unsigned long long bits = 0;
    if (d == 1) {
      mode = CONST;
      if (h) sh.aux[p] = tid;
    } else {
      const unsigned long long raw = section_bytes(RAW, k, n, nseg, 0);
      bool escape = true;
      mode = RAW;
      if (p == 0 && a.group_map) {
        const int g = a.group_map[c];
        const uint8_t gl = tid < A ? a.group_len[g * 256 + tid] : 0;
        const int miss = block_count<DT>(sh, h != 0 && gl == 0);
        if (miss == 0) {
          escape = false;
          bits = block_sum<DT>(sh, (unsigned long long)h * gl);
          if (section_bytes(GROUP, k, n, nseg, bits) < raw) {
            mode = GROUP;
            if (tid < A) {
              sh.len[p][tid] = gl;
              sh.enc[p][tid] = a.group_enc[g * 256 + tid];
            }
            if (tid == 0) sh.aux[p] = g;
          }
        }
      }
      if (escape) {
        if (tid < A) sh.u.cb.hw[tid] = h;
        __syncthreads();
        pm_lengths<ENC_NT>(sh.u.cb.pm, sh.u.cb.hw, A, false, sh.len[p]);
        const uint8_t l = tid < A ? sh.len[p][tid] : 0;
        bits = block_sum<DT>(sh, (unsigned long long)h * l);
        if (section_bytes(HUFF, k, n, nseg, bits) < raw) {
          mode = HUFF;
          canon_encode_table(sh.len[p], A, sh.enc[p], sh.cnt);
        }
      }
      if (mode == RAW) {
        if (tid < A) sh.enc[p][tid] = uint32_t(tid) | (uint32_t(k) << 16);
        bits = uint64_t(n) * k;
      }
      if (tid == 0 && mode != GROUP) sh.aux[p] = 0;
    }
    if (tid == 0) {
      sh.mode[p] = mode;
      sh.bits[p] = bits;
      sh.sec_off[p] = rec;
    }
    rec += section_bytes(mode, k, n, nseg, mode == RAW ? 0 : bits);
    __syncthreads();
  }

  // ------------------------------------------------ 3. decoupled look-back
  if (wv == 0) {
    unsigned long long excl = 0;
    if (ln == 0)
      __hip_atomic_store(&a.status[c], (c == 0 ? FLAG_INC : FLAG_AGG) | rec, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (c > 0) {
      long long top = (long long)c - 1;
      int spins = 0;
      while (true) {
        const long long idx = top - ln;
        unsigned long long st = FLAG_INC;
        if (idx >= 0)
          st = __hip_atomic_load(&a.status[idx], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long fl = st >> 62;
        const unsigned long long inc = __ballot(fl == 2), zero = __ballot(fl == 0);
        const int first = inc ? __ffsll((long long)inc) - 1 : 63;
        const unsigned long long need = first == 63 ? ~0ull : ((2ull << first) - 1);
        if (zero & need) {
          if (++spins > SPIN_LIMIT) {
            if (ln == 0) atomicOr(&a.ctl[0], kErrSpin);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        excl += wave_sum_u64(ln <= first ? (st & VALUE_MASK) : 0ull);
        if (inc) break;
        top -= 64;
      }
    }
    if (ln == 0) {
      __hip_atomic_store(&a.status[c], FLAG_INC | (excl + rec), __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
      sh.excl = excl;
    }
  }
  __syncthreads();
  const uint64_t roff = a.L.off_records + sh.excl;
  if (tid == 0) *reinterpret_cast<uint64_t *>(a.out + a.L.off_dir + 8ull * c) = roff;
  if (roff + rec + 16 > a.cap) {
    if (tid == 0) atomicOr(&a.ctl[0], kErrCapacity);
    return;
  }

  // -------------------------------------------------------- 4. the record
  for (int p = 0; p < NC; p++) {
    const int k = kbits(DT, p), A = 1 << k, mode = sh.mode[p];
    const uint64_t bits = sh.bits[p];
    uint8_t *sec = a.out + roff + sh.sec_off[p];
    const uint64_t head = head_bytes_of(mode, k, nseg);
    const uint64_t pay = payload_bytes_of(mode, k, n, bits);
    // stream header, code lengths and the zero pad of the head
    if (tid == 0) {
      *reinterpret_cast<uint32_t *>(sec) =
          uint32_t(mode) | (uint32_t(sh.aux[p]) << 8) | (uint32_t(nseg) << 16);
      *reinterpret_cast<uint32_t *>(sec + 4) = uint32_t(pay);
    }
    uint64_t used = 8;
    if (mode == HUFF) {
      if (tid < A / 2) sec[8 + tid] = uint8_t(sh.len[p][2 * tid] | (sh.len[p][2 * tid + 1] << 4));
      used += A / 2;
    }
    if (mode == HUFF || mode == GROUP) used += 2ull * nseg;
    for (uint64_t i = used + tid; i < head; i += ENC_NT) sec[i] = 0;
    if (mode == CONST) continue;
    uint32_t *pw = reinterpret_cast<uint32_t *>(sec + head);
    uint16_t *segt = reinterpret_cast<uint16_t *>(sec + 8 + (mode == HUFF ? A / 2 : 0));
    const bool with_segs = mode != RAW;
    uint64_t tbit = 0;     // stream bits before this tile
    uint32_t carry = 0;    // partial last word of the previous tile
    // Huffman-coded streams: wave w of tile T packs segment j = 8T + w, whose
    // symbols are the 32-symbol strips j, j + nseg, ... of the chunk; lane l
    // takes symbols [l*EPT, l*EPT + EPT) of the segment, which lie in one
    // strip.  Raw streams are packed in element order.
    const int ntiles = (nseg + 7) / 8;
    for (int T = 0; T < ntiles; T++) {
      const uint32_t tb = uint32_t(T) * 8u * S;
      const int jseg = T * 8 + wv;
      uint32_t eb;
      bool has = true;
      if (with_segs) {
        const uint32_t si = uint32_t(ln) * EPT;
        eb = 32u * ((si / 32) * uint32_t(nseg) + uint32_t(jseg)) + si % 32;
        has = jseg < nseg;
      } else {
        eb = tb + uint32_t(tid) * EPT;
      }
      if (!has) eb = n;  // no symbols in this lane
      uint32_t w[EPT];
      if (aligned && eb + EPT <= n) {
        const uint8_t *vp = src + uint64_t(eb) * ES;
        u32x4 qs[NV];
#pragma unroll
        for (int j = 0; j < NV; j++) qs[j] = ldg16(vp + 16 * j);
#pragma unroll
        for (int j = 0; j < NV; j++) {
          const uint4 q = make_uint4(qs[j][0], qs[j][1], qs[j][2], qs[j][3]);
#pragma unroll
          for (int i = 0; i < VE; i++) w[j * VE + i] = vec_elem<DT>(q, i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < EPT; i++)
          w[i] = eb + i < n ? load_elem<DT>(src + uint64_t(eb + i) * ES) : 0;
      }
      uint32_t code[EPT];
      int nb = 0;
#pragma unroll
      for (int i = 0; i < EPT; i++) {
        code[i] = eb + i < n ? sh.enc[p][field_rt<DT>(w[i], p)] : 0;
        nb += int(code[i] >> 16);
      }
      const uint32_t incl = wave_incl_scan(uint32_t(nb));
      if (ln == 63) sh.u.pk.wtot[wv] = incl;
      for (int i = tid; i < EncShared<DT>::STAGE; i += ENC_NT) sh.u.pk.stage[i] = 0;
      __syncthreads();
      uint32_t woff = 0, ttot = 0;
      for (int q = 0; q < 8; q++) {
        const uint32_t x = sh.u.pk.wtot[q];
        woff += q < wv ? x : 0;
        ttot += x;
      }
      if (with_segs && ln == 0 && jseg < nseg) stg2(segt + jseg, sh.u.pk.wtot[wv]);
      if (tid == 0 && carry) atomicOr(&sh.u.pk.stage[0], carry);
      const uint32_t start = uint32_t(tbit & 31) + woff + incl - uint32_t(nb);
      uint32_t wi = start >> 5;
      int ab = int(start & 31);
      unsigned long long acc = 0;
#pragma unroll
      for (int i = 0; i < EPT; i++) {
        const int l = int(code[i] >> 16);
        acc |= (unsigned long long)(code[i] & 0xFFFF) << ab;
        ab += l;
        if (ab >= 32) {
          atomicOr(&sh.u.pk.stage[wi], uint32_t(acc));
          wi++;
          acc >>= 32;
          ab -= 32;
        }
      }
      if (ab > 0 && acc) atomicOr(&sh.u.pk.stage[wi], uint32_t(acc));
      __syncthreads();
      const uint32_t endb = uint32_t(tbit & 31) + ttot;
      const uint32_t nfull = endb >> 5;
      const uint64_t w0 = tbit >> 5;
      for (uint32_t i = tid; i < nfull; i += ENC_NT) stg4(pw + w0 + i, sh.u.pk.stage[i]);
      carry = (endb & 31) ? sh.u.pk.stage[nfull] : 0;
      tbit += ttot;
      __syncthreads();
    }
    // last partial word and the zero pad of the payload
    const uint64_t words = (tbit + 31) >> 5;
    if (tid == 0 && (tbit & 31)) pw[tbit >> 5] = carry;
    const uint64_t padw = align16(pay) / 4;
    for (uint64_t i = words + tid; i < padw; i += ENC_NT) pw[i] = 0;
  }
}

__global__ void k_finish(FinishArgs a) {
  const int tid = threadIdx.x;
  for (uint32_t i = tid; i < a.hdr_bytes; i += blockDim.x)
    if (i < 56 || i >= 64) a.out[i] = a.hdr[i];
  uint64_t end = a.L.off_records;
  if (a.L.n_chunks)
    end += a.status[a.L.n_chunks - 1] & VALUE_MASK;
  // zero the alignment gaps around the directory and raw planes
  const uint64_t dir_end = a.L.off_dir + 8ull * (a.L.n_chunks + 1);
  const uint64_t raw0 = a.L.T ? a.L.t_raw[0] : a.L.off_records;
  for (uint64_t i = dir_end + tid; i < raw0; i += blockDim.x) a.out[i] = 0;
  for (int t = tid; t < a.L.T; t += blockDim.x) {
    const uint64_t b = a.L.t_raw[t] + rawplane_bytes(a.dtype, a.L.t_n[t]);
    const uint64_t e = t + 1 < a.L.T ? a.L.t_raw[t + 1] : a.L.off_records;
    for (uint64_t i = b; i < e; i++) a.out[i] = 0;
  }
  if (tid == 0) {
    if (end + 16 > a.cap || (a.ctl[0] & (kErrCapacity | kErrSpin))) {
      atomicOr(&a.ctl[0], kErrCapacity);
    } else {
      *reinterpret_cast<uint64_t *>(a.out + a.L.off_dir + 8ull * a.L.n_chunks) = end;
      *reinterpret_cast<uint64_t *>(a.out + 56) = end + 16;
    }
  }
  if (end + 16 <= a.cap)
    for (int i = tid; i < 16; i += blockDim.x) a.out[end + i] = 0;
}

__global__ void k_zero(uint32_t *p, uint64_t words) {
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < words;
       i += uint64_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

hipError_t launch_encode(int dtype, const EncArgs &a, hipStream_t s) {
  if (a.L.n_chunks == 0) return hipSuccess;
  const dim3 grid(a.L.n_chunks), block(ENC_NT);
  if (dtype == BF16) hipLaunchKernelGGL(k_encode<BF16>, grid, block, 0, s, a);
  else if (dtype == FP32) hipLaunchKernelGGL(k_encode<FP32>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_encode<FP8>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finish(const FinishArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_finish, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero(uint32_t *p, uint64_t words, hipStream_t s) {
  if (!words) return hipSuccess;
  const uint64_t blocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
  hipLaunchKernelGGL(k_zero, dim3(uint32_t(blocks)), dim3(256), 0, s, p, words);
  return hipGetLastError();
}

}  // namespace zn
