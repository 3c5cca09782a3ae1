// zn_common.h -- format constants and workgroup-level code construction for
// the gfx950 codec (libzn.so).  Device code is written for 64-lane wavefronts.
//
// Format (version 1), shared by every kernel here:
//   * field split per element (THEORY-599 on ZipNN, per-field compressibility,
//     ZipNN Table II; FP8: "Lossless Compression of Neural Network Components
//     ... Low-Precision Formats", Abstract):
//       BF16  E = (w>>7)&0xFF coded; SF = sign|frac[6:0] kept raw
//       FP32  P0 = exponent, P1 = sign|frac[22:16], P2, P3 = low fraction
//             bytes, all coded (raw fallback)
//       FP8   E4 = (b>>3)&15, M3 = b&7 coded; sign bit kept raw
//       FP4 pairs (E2M1, two values per byte, the first in the low nibble;
//             a nibble is sign(3) | exponent(2..1) | mantissa(0)):
//             E = e_lo | e_hi<<2 and M = m_lo | m_hi<<1 coded; the two sign
//             bits kept raw
//   * per chunk and coded stream: order-0 histogram, optimal prefix code with
//     lengths <= 11 (package-merge, leaves by (count, symbol), leaves before
//     packages at equal weight), canonical codes, LSB-first bits with each
//     code word first-bit-first (THEORY-599, order-0 only);
//   * streams cut into segments of S symbols (BF16 512, FP32 256, FP8 1024)
//     whose bit lengths are stored, so segments decode independently;
//   * container: 64-byte header, tensor table, chunk directory, raw planes,
//     16-byte aligned chunk records, 16 zero bytes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace zn {

constexpr int kMaxLen = 11;           // longest code word, bits
constexpr int kLutBits = 11;          // decode window = kMaxLen
constexpr int kLutSize = 1 << kLutBits;
constexpr uint32_t kMagic = 0x31464E5Au;     // "ZNF1"
constexpr uint32_t kTsMagic = 0x53544E5Au;   // "ZNTS"
constexpr int kVersion = 1;
constexpr int kRounds = 8;            // Lloyd rounds of the grouped setup

enum Mode { RAW = 0, CONST = 1, HUFF = 2, GROUP = 3, TANS = 4 };
// coder of the exponent stream, chosen per compression call
enum Coder { CODER_HUFFMAN = 0, CODER_TANS = 1 };
// tabled ANS (Duda): 2^11 states, spread with an odd step (every state once)
constexpr int kTansLog = 11;
constexpr uint32_t kTansStates = 1u << kTansLog;
constexpr uint32_t kTansStep = 1283;
enum DType { BF16 = 0, FP32 = 1, FP8 = 2, FP4X2 = 3 };

__host__ __device__ constexpr int esize(int dt) { return dt == BF16 ? 2 : dt == FP32 ? 4 : 1; }
__host__ __device__ constexpr int ncoded(int dt) { return dt == BF16 ? 1 : dt == FP32 ? 4 : 2; }
__host__ __device__ constexpr int kbits(int dt, int p) {
  return dt == FP8 ? (p == 0 ? 4 : 3) : dt == FP4X2 ? (p == 0 ? 4 : 2) : 8;
}
// symbols per segment: a full 256 KiB chunk gives 256 segments per coded stream
__host__ __device__ constexpr int segsyms(int dt) { return dt == BF16 ? 512 : dt == FP32 ? 256 : 1024; }
__host__ __device__ constexpr uint64_t align16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
__host__ __device__ inline uint64_t rawplane_bytes(int dt, uint64_t n) {
  return dt == BF16 ? n : dt == FP8 ? (n + 7) / 8 : dt == FP4X2 ? (n + 3) / 4 : 0;
}
__host__ __device__ inline uint64_t payload_bytes_of(int mode, int k, uint64_t n, uint64_t bits) {
  if (mode == HUFF || mode == GROUP || mode == TANS) return 4 * ((bits + 31) / 32);
  if (mode == RAW) return (n * uint64_t(k) + 7) / 8;
  return 0;
}
// d: symbols present (a TANS head stores a presence mask of 2^k bits and the
// count of each present symbol)
__host__ __device__ inline uint64_t head_bytes_of(int mode, int k, int nseg, int d = 0) {
  uint64_t h = 8;
  if (mode == HUFF) h += uint64_t(1 << k) / 2;
  if (mode == HUFF || mode == GROUP) h += 2 * uint64_t(nseg);
  if (mode == TANS) h += uint64_t(1 << k) / 8 + 2 * uint64_t(d) + 2 * uint64_t(nseg);
  return align16(h);
}
__host__ __device__ inline uint64_t section_bytes(int mode, int k, uint64_t n, int nseg, uint64_t bits,
                                                 int d = 0) {
  return head_bytes_of(mode, k, nseg, d) + align16(payload_bytes_of(mode, k, n, bits));
}

// Global-memory pointers.  Pointers read from device arrays are generic to
// the compiler; casting them to address space 1 gives global_load/store
// (vector memory only, no LDS counter) and lets loads be scheduled early.
#define ZN_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const ZN_GLOBAL T *gptr(const T *p) {
  return (const ZN_GLOBAL T *)(p);
}
template <class T>
__device__ __forceinline__ ZN_GLOBAL T *gptr(T *p) {
  return (ZN_GLOBAL T *)(p);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 ldg16(const void *p) { return *(const ZN_GLOBAL u32x4 *)(p); }
__device__ __forceinline__ u32x2 ldg8(const void *p) { return *(const ZN_GLOBAL u32x2 *)(p); }
__device__ __forceinline__ uint32_t ldg4(const void *p) { return *(const ZN_GLOBAL uint32_t *)(p); }
__device__ __forceinline__ uint32_t ldg2(const void *p) { return *(const ZN_GLOBAL uint16_t *)(p); }
__device__ __forceinline__ uint32_t ldg1(const void *p) { return *(const ZN_GLOBAL uint8_t *)(p); }
// Streaming loads of data read once: the non-temporal hint keeps them from
// displacing reused lines in the caches.
__device__ __forceinline__ u32x4 ldg16s(const void *p) {
  return __builtin_nontemporal_load((const ZN_GLOBAL u32x4 *)(p));
}
__device__ __forceinline__ u32x2 ldg8s(const void *p) {
  return __builtin_nontemporal_load((const ZN_GLOBAL u32x2 *)(p));
}
__device__ __forceinline__ void stg16(void *p, u32x4 v) { *(ZN_GLOBAL u32x4 *)(p) = v; }
// Streaming store of output read by nothing here: the non-temporal hint
// writes it through instead of leaving dirty lines for later kernels to evict.
__device__ __forceinline__ void stg16s(void *p, u32x4 v) { __builtin_nontemporal_store(v, (ZN_GLOBAL u32x4 *)(p)); }
__device__ __forceinline__ void stg8(void *p, u32x2 v) { *(ZN_GLOBAL u32x2 *)(p) = v; }
__device__ __forceinline__ void stg4(void *p, uint32_t v) { *(ZN_GLOBAL uint32_t *)(p) = v; }
__device__ __forceinline__ void stg2(void *p, uint32_t v) { *(ZN_GLOBAL uint16_t *)(p) = uint16_t(v); }
__device__ __forceinline__ void stg1(void *p, uint32_t v) { *(ZN_GLOBAL uint8_t *)(p) = uint8_t(v); }

// Plan tables that kernels read (device memory owned by the tableset).
struct DevLayout {
  const uint64_t *t_n;       // [T] elements per tensor
  const uint64_t *t_raw;     // [T] offset of the tensor's always-raw section
  const uint32_t *t_chunk0;  // [T+1] first global chunk of each tensor
  int T;
  uint32_t n_chunks;
  uint32_t chunk_elems;
  uint64_t off_dir, off_records;
};

__device__ inline int find_tensor(const DevLayout &L, uint32_t c) {
  int lo = 0, hi = L.T - 1;  // last t with t_chunk0[t] <= c
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (L.t_chunk0[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- waves ----
__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline uint64_t lanemask_lt() {
  const int ln = threadIdx.x & 63;
  return ln ? (~0ull >> (64 - ln)) : 0ull;
}
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then row_bcast:15 adds
// row 0's (row 2's) total to row 1 (row 3), and row_bcast:31 adds lane 31's
// running total to rows 2 and 3.  Lanes without a source receive 0.
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  int x = int(v);
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return uint32_t(x);
}

// ------------------------------------------------------- package-merge ----
// Shared memory of one code construction over at most AM symbols (about
// 18 KB for 256, 33 KB for 512).
template <int AM>
struct PMSharedA {
  using Sym = std::conditional_t<(AM > 256), uint16_t, uint8_t>;
  uint64_t w[2][2 * AM];            // item weights of the previous/current list
  uint64_t leaf_w[AM];              // leaves sorted by (count, symbol)
  Sym leafcl[kMaxLen][AM];          // packages ahead of sorted leaf i in list j
  Sym leaf_sym[AM];
  Sym tmp_sym[AM];
  int c[kMaxLen];                   // leaves among the selected prefix of list j
  int d;
  int wave_cnt[AM / 64];
};
using PMShared = PMSharedA<256>;
// present symbols in symbol order, before sorting (shares w[1], which is
// written only from the first merge on)
#define PM_TMP_W(S) ((S).w[1])

// Optimal code lengths (<= 11) of the weights hw[0..A) by package-merge, for
// a workgroup of NT >= 256 threads.  List 0 holds the leaves (coins of the
// smallest denomination); list j merges leaves with packages made of adjacent
// pairs of list j-1, leaves first at equal weight; the first 2d-2 items of
// the last list are selected.  Instead of expanding packages, the number of
// leaves c_j inside the selected prefix of each list is counted backwards
// (a prefix of p packages is exactly the first 2p items of the list below),
// and sorted leaf i gets the length #{j : i < c_j}.
// Returns d, the number of symbols with non-zero weight (after the group
// rule, which adds the smallest absent symbol with weight 0 when d == 1).
// len[0..A) is written for every symbol (0 when absent).
template <int NT, int AM = 256>
__device__ int pm_lengths(PMSharedA<AM> &S, const uint64_t *hw, int A, bool group_rule, uint8_t *len) {
  static_assert(NT >= AM, "code construction needs a thread per symbol");
  using Sym = typename PMSharedA<AM>::Sym;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  const bool nz = tid < A && hw[tid] != 0;
  const uint64_t m = __ballot(nz);
  if (ln == 0 && wv < AM / 64) S.wave_cnt[wv] = __popcll(m);
  if (tid < A) len[tid] = 0;
  __syncthreads();
  if (nz) {
    int base = 0;
    for (int q = 0; q < wv; q++) base += S.wave_cnt[q];
    const int idx = base + __popcll(m & lanemask_lt());
    S.tmp_sym[idx] = Sym(tid);
    PM_TMP_W(S)[idx] = hw[tid];
  }
  if (tid == 0) {
    int d = 0;
    for (int q = 0; q < AM / 64; q++) d += S.wave_cnt[q];
    S.d = d;
  }
  __syncthreads();
  int d = S.d;
  if (group_rule && d == 1) {
    if (tid == 0) {
      S.tmp_sym[1] = S.tmp_sym[0] == 0 ? 1 : 0;
      PM_TMP_W(S)[1] = 0;
      S.d = 2;
    }
    __syncthreads();
    d = 2;
  }
  if (d < 2) return d;
  // rank sort of the leaves by (weight, symbol)
  if (tid < d) {
    const uint64_t w = PM_TMP_W(S)[tid];
    const int s = S.tmp_sym[tid];
    int r = 0;
    for (int j = 0; j < d; j++) {
      const uint64_t wj = PM_TMP_W(S)[j];
      r += (wj < w) || (wj == w && S.tmp_sym[j] < s);
    }
    S.leaf_w[r] = w;
    S.leaf_sym[r] = Sym(s);
    S.w[0][r] = w;
    S.leafcl[0][r] = 0;
  }
  __syncthreads();
  int n_prev = d;
  for (int j = 1; j < kMaxLen; j++) {
    const uint64_t *prev = S.w[(j - 1) & 1];
    uint64_t *cur = S.w[j & 1];
    const int np = n_prev >> 1;
    for (int q = tid; q < d + np; q += NT) {
      if (q < d) {  // leaf q: after every package lighter than it
        const uint64_t wi = S.leaf_w[q];
        int lo = 0, hi = np;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (prev[2 * mid] + prev[2 * mid + 1] < wi) lo = mid + 1; else hi = mid;
        }
        cur[q + lo] = wi;
        S.leafcl[j][q] = Sym(lo);
      } else {      // package k: after every leaf not heavier than it
        const int k = q - d;
        const uint64_t p = prev[2 * k] + prev[2 * k + 1];
        int lo = 0, hi = d;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (S.leaf_w[mid] <= p) lo = mid + 1; else hi = mid;
        }
        cur[k + lo] = p;
      }
    }
    __syncthreads();
    n_prev = d + np;
  }
  if (tid < 64) {
    int msel = 2 * d - 2;
    for (int j = kMaxLen - 1; j >= 0; j--) {
      int cnt = 0;
      for (int i = tid; i < d; i += 64) cnt += i + S.leafcl[j][i] < msel;
      cnt = wave_sum(cnt);
      if (tid == 0) S.c[j] = cnt;
      msel = 2 * (msel - cnt);
    }
  }
  __syncthreads();
  if (tid < d) {
    int l = 0;
    for (int j = 0; j < kMaxLen; j++) l += tid < S.c[j];
    len[S.leaf_sym[tid]] = uint8_t(l);
  }
  __syncthreads();
  return d;
}

// ------------------------------------------- one-wave code construction ----
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), lane));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), lane));
  return lo | (uint64_t(hi) << 32);
}
__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Orders this wave's LDS writes before its later LDS reads by other lanes of
// the same wave.  The hardware already runs a wave's LDS instructions in
// order; the wavefront-scope release/acquire fences are what stop the
// compiler from moving the memory operations of one lane across the point
// (the wave barrier alone does not: it is not a memory operation).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave-private LDS of the one-wave package-merge.
struct WaveCB {
  uint64_t lst[128];   // the current merged list
  uint64_t srt[64];    // present symbols' counts, in symbol order
  uint64_t leaf[64];   // leaf weights sorted by (count, symbol)
  uint64_t pk[64];     // the packages of the list being built
  uint8_t sym[64], ssym[64];
};

// The package-merge of pm_lengths (same lists, same tie rule, same result)
// run by one wave when at most 64 symbols are present: leaf i lives in lane
// i, list item j in lane j (j < 64) or lane j-64.  Both inputs of each merge
// are sorted, so each item's rank in the merged list comes from a binary
// search of the other input in LDS; no workgroup barrier is needed.
// Returns d (after the group rule), or -1 when more than 64 symbols are
// present (the workgroup version must run).  Every lane of the wave calls it.
template <class WT>
__device__ int wave_pm_lengths(const WT *hist, int A, bool group_rule, uint8_t *len, WaveCB &W) {
  const int ln = threadIdx.x & 63;
  uint64_t x[4], m[4];
  int d = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int s = ln + 64 * q;
    x[q] = s < A ? uint64_t(hist[s]) : 0;
    m[q] = __ballot(x[q] != 0);
    d += __popcll(m[q]);
    if (s < A) len[s] = 0;
  }
  if (d > 64) return -1;
  int base = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if (x[q]) {
      const int idx = base + __popcll(m[q] & lanemask_lt());
      W.srt[idx] = x[q];
      W.sym[idx] = uint8_t(ln + 64 * q);
    }
    base += __popcll(m[q]);
  }
  wave_lds_sync();
  if (group_rule && d == 1) {
    if (ln == 0) {
      W.sym[1] = W.sym[0] == 0 ? 1 : 0;
      W.srt[1] = 0;
    }
    wave_lds_sync();
    d = 2;
  }
  if (d < 2) return d;
  // rank sort of the leaves by (weight, symbol)
  const uint64_t w = ln < d ? W.srt[ln] : ~0ull;
  const int sy = ln < d ? W.sym[ln] : 255;
  int r = 0;
  for (int j = 0; j < d; j++) {
    const uint64_t wj = readlane64(w, j);
    const int sj = __builtin_amdgcn_readlane(sy, j);
    r += (wj < w) || (wj == w && sj < sy);
  }
  wave_lds_sync();
  if (ln < d) {
    W.lst[r] = w;
    W.ssym[r] = uint8_t(sy);
  }
  wave_lds_sync();
  const uint64_t lw = ln < d ? W.lst[ln] : ~0ull;
  const int lsym = ln < d ? W.ssym[ln] : 0;
  if (ln < d) W.leaf[ln] = lw;
  uint64_t c0 = lw, c1 = 0;
  int ncur = d;
  int lp[kMaxLen];
  lp[0] = ln;
#pragma unroll
  for (int j = 1; j < kMaxLen; j++) {
    const int np = ncur >> 1;
    const int i0 = 2 * ln, i1 = 2 * ln + 1;
    const uint64_t a0 = __shfl(c0, i0 & 63, 64), a1 = __shfl(c1, i0 & 63, 64);
    const uint64_t b0 = __shfl(c0, i1 & 63, 64), b1 = __shfl(c1, i1 & 63, 64);
    const uint64_t P = (i0 < 64 ? a0 : a1) + (i1 < 64 ? b0 : b1);
    if (ln < np) W.pk[ln] = P;
    wave_lds_sync();
    // cl = packages lighter than the leaf, cp = leaves not heavier than the
    // package (leaves go first at equal weight): binary lifting over <= 64
    int cl = 0, cp = 0;
#pragma unroll
    for (int step = 64; step; step >>= 1) {
      const int a = cl + step, b = cp + step;
      const uint64_t pa = W.pk[(a <= np ? a : 1) - 1], lb = W.leaf[(b <= d ? b : 1) - 1];
      cl = a <= np && pa < lw ? a : cl;
      cp = b <= d && lb <= P ? b : cp;
    }
    wave_lds_sync();
    if (ln < d) W.lst[ln + cl] = lw;
    if (ln < np) W.lst[ln + cp] = P;
    lp[j] = ln + cl;
    wave_lds_sync();
    ncur = d + np;
    c0 = ln < ncur ? W.lst[ln] : 0;
    c1 = ln + 64 < ncur ? W.lst[ln + 64] : 0;
  }
  int msel = 2 * d - 2, l = 0;
#pragma unroll
  for (int j = kMaxLen - 1; j >= 0; j--) {
    const int cnt = __popcll(__ballot(ln < d && lp[j] < msel));
    l += ln < cnt;
    msel = 2 * (msel - cnt);
  }
  if (ln < d) len[lsym] = uint8_t(l);
  wave_lds_sync();
  return d;
}

// Canonical codes (RFC 1951 section 3.2.2) by one wave: enc[s] = bit-reversed
// code | (length << 16), for A <= 256 symbols.
__device__ inline void wave_canon(const uint8_t *len, int A, uint32_t *enc) {
  const int ln = threadIdx.x & 63;
  int l[4], rank[4] = {0, 0, 0, 0};
  uint32_t bl[kMaxLen + 1];
  bl[0] = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) l[q] = ln + 64 * q < A ? len[ln + 64 * q] : 0;
#pragma unroll
  for (int b = 1; b <= kMaxLen; b++) {
    int base = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint64_t mm = __ballot(l[q] == b);
      if (l[q] == b) rank[q] = base + __popcll(mm & lanemask_lt());
      base += __popcll(mm);
    }
    bl[b] = uint32_t(base);
  }
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int s = ln + 64 * q;
    if (s >= A) continue;
    uint32_t e = 0;
    if (l[q]) {
      uint32_t code = 0;
#pragma unroll
      for (int b = 1; b <= kMaxLen; b++)
        if (b <= l[q]) code = (code + bl[b - 1]) << 1;
      code += uint32_t(rank[q]);
      e = (__builtin_bitreverse32(code) >> (32 - l[q])) | (uint32_t(l[q]) << 16);
    }
    enc[s] = e;
  }
  wave_lds_sync();
}

// ------------------------------------------------------ canonical codes ----
// Canonical code values (RFC 1951 section 3.2.2) of lengths len[0..A),
// stored for LSB-first emission: enc[s] = bit-reversed code | (length << 16).
// cnt: shared [4][kMaxLen + 1].  Any NT >= 256.
__device__ inline void canon_encode_table(const uint8_t *len, int A, uint32_t *enc,
                                          int (*cnt)[kMaxLen + 1]) {
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  const int l = tid < A ? len[tid] : 0;
  int rank = 0;
  for (int b = 1; b <= kMaxLen; b++) {
    const uint64_t m = __ballot(l == b);
    if (l == b) rank = __popcll(m & lanemask_lt());
    if (ln == 0 && wv < 4) cnt[wv][b] = __popcll(m);
  }
  __syncthreads();
  if (tid < A) {
    uint32_t e = 0;
    if (l) {
      uint32_t code = 0;
      for (int b = 1; b <= l; b++) {
        const int prevc = b > 1 ? cnt[0][b - 1] + cnt[1][b - 1] + cnt[2][b - 1] + cnt[3][b - 1] : 0;
        code = (code + prevc) << 1;
      }
      for (int q = 0; q < wv; q++) code += cnt[q][l];
      code += rank;
      e = (__builtin_bitreverse32(code) >> (32 - l)) | (uint32_t(l) << 16);
    }
    enc[tid] = e;
  }
  __syncthreads();
}

// ------------------------------------------------------ decode tables ------
// Shared memory for one decode table build.
struct LutShared {
  int cnt[4][kMaxLen + 1];
  int first[kMaxLen + 2];     // first canonical code of each length
  int offs[kMaxLen + 2];      // sorted index of the first symbol of each length
  int ljend[kMaxLen + 2];     // end of each length's range, left-justified to 11 bits
  uint8_t sorted[256];        // symbols ordered by (length, symbol)
  int bad;
};

// Builds the multi-symbol decode table of a canonical code from its lengths.
// lut[v] for a WB-bit LSB-first window v (2^WB entries) holds up to three
// whole code words: bits 0-5 the bits they use (so the entry itself can serve
// as a shift amount), 6-7 their number, 8-15, 16-23, 24-31 the symbols.  t1
// (2^WB x u16, scratch) is the single-symbol table, indexed like lut by the
// LSB-first window: symbol | length << 8.  Returns false (for every thread) if
// the lengths are not a complete prefix code of at least two words with
// lengths <= min(11, WB).  A window narrower than 11 bits serves small
// alphabets: a complete code over d symbols has no word longer than d - 1
// bits.  NT >= 256 threads; A <= 256.
template <int NT, int WB = kLutBits>
__device__ __attribute__((always_inline)) bool build_lut(const uint8_t *len, int A, uint32_t *lut, uint16_t *t1,
                                                     LutShared &S) {
  static_assert(WB >= 2 && WB <= kLutBits, "window of 2..11 bits");
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  const int l = tid < A ? len[tid] : 0;
  int rank = 0;
  for (int b = 1; b <= kMaxLen; b++) {
    const uint64_t m = __ballot(l == b);
    if (l == b) rank = __popcll(m & lanemask_lt());
    if (ln == 0 && wv < 4) S.cnt[wv][b] = __popcll(m);
  }
  if (tid == 0) S.bad = 0;
  __syncthreads();
  if (tid < A && l > (WB < kMaxLen ? WB : kMaxLen)) S.bad = 1;
  if (wv == 0) {
    // lane b (1..11): the number of codes of length b, the sorted index of
    // the first of them, the first canonical code of length b (the sum of
    // c_j << (b - j) over j < b) and the end of its range left-justified
    const int b = ln;
    const bool isb = b >= 1 && b <= kMaxLen;
    const int c = isb ? S.cnt[0][b] + S.cnt[1][b] + S.cnt[2][b] + S.cnt[3][b] : 0;
    const uint32_t incl = wave_incl_scan(uint32_t(c));
    uint32_t first = 0;
#pragma unroll
    for (int j = 1; j < kMaxLen; j++) {
      const uint32_t cj = uint32_t(__builtin_amdgcn_readlane(c, j));
      first += j < b ? cj << (b - j) : 0u;
    }
    const uint32_t kr = wave_incl_scan(isb ? uint32_t(c) << (kMaxLen - (isb ? b : 1)) : 0u);
    const uint32_t kraft = uint32_t(__builtin_amdgcn_readlane(int(kr), 63));
    const uint32_t d = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
    if (isb) {
      S.first[b] = int(first);
      S.offs[b] = int(incl) - c;
      S.ljend[b] = int((first + uint32_t(c)) << (kMaxLen - b));
    }
    if (ln == 0 && (d < 2 || kraft != (1u << kMaxLen))) S.bad = 1;
  }
  __syncthreads();
  if (S.bad) return false;
  if (tid < A && l) {
    int pos = S.offs[l] + rank;
    for (int q = 0; q < wv; q++) pos += S.cnt[q][l];
    S.sorted[pos] = uint8_t(tid);
  }
  __syncthreads();
  // single-symbol table: the length of the code starting a window is one
  // more than the number of lengths whose range ends at or below it.
  // Counted with subtract-and-shift in inline asm: as compares they would
  // all write one condition register and serialise the entries of a thread.
  // All lengths first, then all table reads, then all writes, so that the
  // reads of the eight entries of a thread overlap.
  constexpr int TS = 1 << WB;                  // table entries
  static_assert(TS % NT == 0 || TS < NT, "whole passes");
  constexpr int PER = TS >= NT ? TS / NT : 1;  // entries per thread (threads past TS idle)
  const bool own = tid < TS;
  int ljm[kMaxLen];
#pragma unroll
  for (int j = 1; j < kMaxLen; j++) ljm[j] = S.ljend[j] - 1;
  // Entry v of t1 is the code starting the LSB-first window v, whose
  // first-bit-as-MSB reading u = reverse(v) is what the ranges compare.
  // Threads take consecutive v, so both the stores here and the first
  // lookups below fall in distinct LDS banks.
  // (reading the window's WB bits as the top bits of an 11-bit code)
  auto rev11 = [](int v) {
    return int(__builtin_bitreverse32(uint32_t(v)) >> (32 - WB)) << (kMaxLen - WB);
  };
  auto win = [&](int i) { return (tid + i * NT) & (TS - 1); };   // this thread's i-th window
  int bl[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int u = rev11(win(i));
    int b = 1;
#pragma unroll
    for (int j = 1; j < kMaxLen; j++) {
      int ge;   // 1 if u >= ljend[j]
      asm("v_sub_u32 %0, %1, %2\n\tv_lshrrev_b32 %0, 31, %0" : "=&v"(ge) : "v"(ljm[j]), "v"(u));
      b += ge;
    }
    bl[i] = b;
  }
  int fo[PER], of[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    fo[i] = S.first[bl[i]];
    of[i] = S.offs[bl[i]];
  }
  uint32_t tv[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int u = rev11(win(i));
    tv[i] = uint32_t(S.sorted[of[i] + (u >> (kMaxLen - bl[i])) - fo[i]]) | uint32_t(bl[i] << 8);
  }
#pragma unroll
  for (int i = 0; i < PER; i++)
    if (own) t1[win(i)] = uint16_t(tv[i]);
  __syncthreads();
  // up to three whole code words per window, without branches; the three
  // lookups of the entries of a thread go in three passes
  auto t1at = [&](uint32_t w) { return uint32_t(t1[w]); };
  uint32_t e1[PER], e2[PER], e3[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) e1[i] = t1at(uint32_t(win(i)));
#pragma unroll
  for (int i = 0; i < PER; i++) e2[i] = t1at(uint32_t(win(i)) >> (e1[i] >> 8));
#pragma unroll
  for (int i = 0; i < PER; i++) e3[i] = t1at((uint32_t(win(i)) >> (e1[i] >> 8)) >> (e2[i] >> 8));
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const uint32_t l1 = e1[i] >> 8, l2 = e2[i] >> 8, l3 = e3[i] >> 8;
    // all-ones masks: the second (third) word fits in the window
    const uint32_t m2 = uint32_t(int(l1 + l2 - WB - 1) >> 31);
    const uint32_t m3 = m2 & uint32_t(int(l1 + l2 + l3 - WB - 1) >> 31);
    const uint32_t used = l1 + (l2 & m2) + (l3 & m3);
    const uint32_t n = 1 + (m2 & 1) + (m3 & 1);
    const uint32_t syms = (e1[i] & 0xFF) | (((e2[i] & 0xFF) << 8) & m2) | (((e3[i] & 0xFF) << 16) & m3);
    tv[i] = used | (n << 6) | (syms << 8);
  }
#pragma unroll
  for (int i = 0; i < PER; i++)
    if (own) lut[win(i)] = tv[i];
  __syncthreads();
  return true;
}

// ------------------------------------------------------------- tANS ----
// The exponent coder of THEORY-599's order-0 discussion (ZipNN Fig. 4: a
// finite-state-entropy coder, i.e. tabled asymmetric numeral systems, codes
// exponents 0-2% smaller than Huffman), after Duda's tabled ANS:
//   * counts q[s] normalised to sum 2^11: floor(h*2^11/n), at least 1 for a
//     present symbol; a shortfall goes one each to the present symbols of
//     largest remainder h*2^11 mod n (ties to the smaller symbol), an excess
//     is taken one at a time from the largest count (ties to the smaller);
//   * the i-th state handed out (symbols in increasing order, q[s] each) is
//     state i*1283 mod 2^11;
//   * a state x holding s has rank r among the states of s below it; decoding
//     x outputs s, forms y = q[s] + r, reads nb = 11 - floor(log2 y) bits v
//     (value bit 0 first) and goes to state (y << nb) + v - 2^11; encoding,
//     backwards from state 2^11 (x = 0), emits the nb low bits of X = 2^11 + x
//     with X >> nb in [q, 2q) and goes to the (X >> nb) - q -th state of s.

// Workgroup LDS of the table construction.
template <int NT>
struct TansBuild {
  uint8_t spread[kTansStates];      // symbol of each state
  uint16_t cnt[NT / 64][256];       // states of each symbol met by each wave
  uint16_t cum[260];                // first assignment index of each symbol
  int ok;
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t t = uint32_t(__shfl_xor(int(v), o, 64));
    v = t > v ? t : v;
  }
  return v;
}

// Normalised counts q[0..A) of the histogram hist[0..A) of n > 0 symbols
// (n <= 2^20, so h * 2^11 fits 32 bits), by one whole wave.  Returns the
// number of present symbols.
__device__ inline int wave_tans_normalize(const uint32_t *hist, int A, uint32_t n, uint32_t *q) {
  const int ln = threadIdx.x & 63;
  uint32_t h[4], c[4], rem[4];
  bool given[4];
  uint32_t part = 0;
  int dl = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int s = ln + 64 * j;
    h[j] = s < A ? hist[s] : 0u;
    const uint32_t x = h[j] * kTansStates;
    const uint32_t f = x / n;
    c[j] = h[j] ? (f ? f : 1u) : 0u;
    rem[j] = h[j] ? x - f * n : 0u;
    given[j] = false;
    part += c[j];
    dl += h[j] != 0;
  }
  int sum = wave_sum(int(part));
  const int d = wave_sum(dl);
  // shortfall: the present symbols of largest remainder, one each (a key is
  // remainder << 8 | (255 - s), plus one so that 0 means none)
  while (sum < int(kTansStates)) {
    uint32_t key = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t kj = (h[j] && !given[j]) ? ((rem[j] << 8) | uint32_t(255 - (ln + 64 * j))) + 1u : 0u;
      key = kj > key ? kj : key;
    }
    key = wave_max_u32(key);
    if (!key) break;   // no symbol left: cannot happen, the floors lose less than one each
    const int s = 255 - int((key - 1u) & 255u);
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (s == ln + 64 * j) {
        c[j]++;
        given[j] = true;
      }
    sum++;
  }
  // excess (symbols raised to 1): one at a time from the largest count
  while (sum > int(kTansStates)) {
    uint32_t key = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t kj = c[j] > 1 ? (c[j] << 8) | uint32_t(255 - (ln + 64 * j)) : 0u;
      key = kj > key ? kj : key;
    }
    key = wave_max_u32(key);
    if (!key) break;   // cannot happen: the excess is at most the symbols raised to 1
    const int s = 255 - int(key & 255u);
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (s == ln + 64 * j) c[j]--;
    sum--;
  }
#pragma unroll
  for (int j = 0; j < 4; j++)
    if (ln + 64 * j < A) q[ln + 64 * j] = c[j];
  return d;
}

// The state tables of the counts q[0..A) (in LDS), by the whole workgroup of
// NT threads.  Writes, where the pointer is not null:
//   dec[x]   = s | nb << 8 | ((y << nb) - 2^11) << 12 for each state x (decoding);
//   est[cum[s] + r] = x, the r-th state of s in increasing order (encoding);
//   esym[s]  = q | nb0 << 12 | (cum - q + 2^11) << 16, nb0 = 11 - floor(log2 q)
//              (0 for an absent symbol).
// Returns false (uniformly) unless the counts sum to 2^11.
template <int NT>
__device__ bool tans_tables(const uint32_t *q, int A, TansBuild<NT> &B, uint32_t *dec, uint16_t *est,
                            uint32_t *esym) {
  constexpr int NW = NT / 64, SPW = int(kTansStates) / NW, PER = int(kTansStates) / NT;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  if (wv == 0) {
    // cumulative counts: lane ln sums symbols 4 ln .. 4 ln + 3
    uint32_t c4[4], part = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int s = 4 * ln + j;
      c4[j] = s < A ? q[s] : 0u;
      part += c4[j];
    }
    const uint32_t incl = wave_incl_scan(part);
    uint32_t run = incl - part;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int s = 4 * ln + j;
      if (s < A) B.cum[s] = uint16_t(run > 0xFFFFu ? 0xFFFFu : run);
      run += c4[j];
    }
    const uint32_t total = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
    if (ln == 0) {
      B.cum[A] = uint16_t(total > 0xFFFFu ? 0xFFFFu : total);
      B.ok = total == kTansStates;
    }
  }
  for (int i = tid; i < NW * 256; i += NT) (&B.cnt[0][0])[i] = 0;
  __syncthreads();
  if (!B.ok) return false;
  // spread: assignment index i goes to state i*1283 mod 2^11
  {
    const int i0 = tid * PER;
    int lo = 0, hi = A - 1;   // last s with cum[s] <= i0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (B.cum[mid] <= i0) lo = mid; else hi = mid - 1;
    }
    int s = lo;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int i = i0 + k;
      while (B.cum[s + 1] <= i) s++;
      B.spread[(uint32_t(i) * kTansStep) & (kTansStates - 1)] = uint8_t(s);
    }
  }
  __syncthreads();
  // ranks: wave wv takes states [wv*SPW, (wv+1)*SPW) in batches of 64; a
  // lane's rank within the wave is the wave's running count of its symbol
  // plus the lanes below it holding the same symbol
  constexpr int NB = SPW / 64;
  uint32_t rl[NB], sy[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const int x = wv * SPW + b * 64 + ln;
    const uint32_t s = B.spread[x];
    uint64_t eq = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 8; bit++) {
      const uint64_t m = __ballot((s >> bit) & 1);
      eq &= ((s >> bit) & 1) ? m : ~m;
    }
    const uint32_t below = uint32_t(__popcll(eq & lanemask_lt()));
    sy[b] = s;
    rl[b] = B.cnt[wv][s] + below;
    wave_lds_sync();
    if (below == 0) B.cnt[wv][s] = uint16_t(B.cnt[wv][s] + __popcll(eq));
    wave_lds_sync();
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const int x = wv * SPW + b * 64 + ln;
    const uint32_t s = sy[b];
    uint32_t r = rl[b];
    for (int w = 0; w < wv; w++) r += B.cnt[w][s];
    const uint32_t qs = q[s];
    if (dec) {
      const uint32_t y = qs + r;                       // in [q, 2q)
      const uint32_t nb = uint32_t(kTansLog) - (31u - uint32_t(__clz(int(y))));
      dec[x] = s | (nb << 8) | (((y << nb) - kTansStates) << 12);
    }
    if (est) est[B.cum[s] + r] = uint16_t(x);
  }
  if (esym && tid < A) {
    const uint32_t qs = q[tid];
    const uint32_t nb0 = qs ? uint32_t(kTansLog) - (31u - uint32_t(__clz(int(qs)))) : 0u;
    esym[tid] = qs ? qs | (nb0 << 12) | ((uint32_t(B.cum[tid]) - qs + kTansStates) << 16) : 0u;
  }
  __syncthreads();
  return true;
}

// One encoding step from state X in [2^11, 2^12) for the symbol whose esym
// entry is info: emits the nb low bits of X (returned: nb, and the bits in v)
// and moves X on.
__device__ __forceinline__ uint32_t tans_enc_step(uint32_t &X, uint32_t info, const uint16_t *est, uint32_t &v) {
  const uint32_t qs = info & 0xFFFu, nb0 = (info >> 12) & 15u;
  const uint32_t nb = nb0 - (X < (qs << nb0) ? 1u : 0u);
  v = X & ((1u << nb) - 1u);
  X = kTansStates + est[(X >> nb) + (info >> 16) - kTansStates];
  return nb;
}

}  // namespace zn
