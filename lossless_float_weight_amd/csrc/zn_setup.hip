// zn_setup.hip -- kernels of the reusable setup ("NeuralZip: Reusable Setup
// for Fast Lossless Compression", Abstract: chunks with similar exponent
// distributions are grouped and share one Huffman code, chosen once before
// later encodings).  All arithmetic is integer, so the grouping equals the
// CPU oracle's exactly:
//   k_hist_all     order-0 histograms of every coded stream of every chunk
//                  (single-step checks)
//   k_hist0        order-0 histogram of the exponent stream of every chunk
//   k_keys         key = floor(sum(s * h[s]) * 2^16 / n) of each chunk
//   k_pool         pooled histogram of each group
//   k_lengths      optimal lengths (<= 11) of a histogram, one per workgroup
//   k_group_tables encode table and decode table of each group
//   k_assign       each chunk to the group code of least coded size
// and, for packed exponent pairs ("NeuralZip", Abstract: recurring exponent
// tuples represented by packed exponents, chosen by the setup):
//   k_pair_F       each group's 16 most common values (F) and their ranks
//   k_pair_tokens  each group's token counts: pairs of values of F at the
//                  aligned positions of each 32-value strip, singles otherwise
//   k_token_lengths optimal lengths (<= 11) over the 512 tokens of a group
//   k_pair_decide  a group packs when its tokens take fewer pooled bits
//   k_pair_tables  encode tables and a one-token decode table of a packing group
#include "zn_internal.h"

namespace zn {

constexpr int HIST_NT = 256;

template <int DT, int P>
__device__ __forceinline__ uint32_t sfield(uint32_t w) {
  if constexpr (DT == BF16) return (w >> 7) & 0xFF;
  if constexpr (DT == FP32) {
    if constexpr (P == 0) return (w >> 23) & 0xFF;
    if constexpr (P == 1) return ((w >> 24) & 0x80) | ((w >> 16) & 0x7F);
    if constexpr (P == 2) return (w >> 8) & 0xFF;
    return w & 0xFF;
  }
  if constexpr (DT == FP4X2) {
    if constexpr (P == 0) return ((w >> 1) & 3) | ((w >> 3) & 0xC);
    return (w & 1) | ((w >> 3) & 2);
  }
  if constexpr (P == 0) return (w >> 3) & 0xF;
  return w & 7;
}

template <int DT>
__device__ __forceinline__ void count_elem(uint32_t *priv, uint32_t w, int col) {
  constexpr int NC = ncoded(DT);
  // bins are laid out [stream][256][32 columns]; column = lane & 31
  atomicAdd(&priv[(0 * 256 + sfield<DT, 0>(w)) * 32 + col], 1u);
  if constexpr (NC > 1) atomicAdd(&priv[(1 * 256 + sfield<DT, 1>(w)) * 32 + col], 1u);
  if constexpr (NC > 2) atomicAdd(&priv[(2 * 256 + sfield<DT, 2>(w)) * 32 + col], 1u);
  if constexpr (NC > 3) atomicAdd(&priv[(3 * 256 + sfield<DT, 3>(w)) * 32 + col], 1u);
}

// One workgroup per chunk; hist[c][NC][256]; bins privatised per lane column
// (FP32's four streams take 128 KB of LDS; this is a one-off setup pass).
template <int DT>
__global__ __launch_bounds__(HIST_NT) void k_hist_all(DevLayout L, const uint8_t *const *in_ptrs,
                                                      uint32_t *hist) {
  constexpr int NC = ncoded(DT), ES = esize(DT);
  __shared__ uint32_t priv[NC * 256 * 32];
  const int tid = threadIdx.x, col = tid & 31;
  const uint32_t c = blockIdx.x;
  const int t = find_tensor(L, c);
  const uint64_t e0 = uint64_t(c - L.t_chunk0[t]) * L.chunk_elems;
  const uint64_t rem = L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < L.chunk_elems ? rem : L.chunk_elems);
  const uint8_t *src = in_ptrs[t] + e0 * ES;
  for (int i = tid; i < NC * 256 * 32; i += HIST_NT) priv[i] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < n; i += HIST_NT) {
    const uint8_t *p = src + uint64_t(i) * ES;
    uint32_t w = p[0];
    if constexpr (ES >= 2) w |= uint32_t(p[1]) << 8;
    if constexpr (ES == 4) w |= (uint32_t(p[2]) << 16) | (uint32_t(p[3]) << 24);
    count_elem<DT>(priv, w, col);
  }
  __syncthreads();
  for (int i = tid; i < NC * 256; i += HIST_NT) {
    uint32_t s = 0;
    for (int j = 0; j < 32; j++) s += priv[i * 32 + ((j + i) & 31)];
    hist[uint64_t(c) * NC * 256 + i] = s;
  }
}

// Order-0 histogram of the first coded stream (the exponent) of every chunk,
// the only one the grouping reads: hist[c][256].  One workgroup per chunk
// reads it with 16-byte loads (a byte at a time only for a ragged tail or
// unaligned input) and counts in LDS bins privatised per lane column.
template <int DT>
__global__ __launch_bounds__(HIST_NT) void k_hist0(DevLayout L, const uint8_t *const *in_ptrs, uint32_t *hist) {
  constexpr int ES = esize(DT), VE = 16 / ES, COLS = 32;
  __shared__ uint32_t priv[256 * COLS];
  const int tid = threadIdx.x, col = tid & (COLS - 1);
  const uint32_t c = blockIdx.x;
  const int t = find_tensor(L, c);
  const uint64_t e0 = uint64_t(c - L.t_chunk0[t]) * L.chunk_elems;
  const uint64_t rem = L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < L.chunk_elems ? rem : L.chunk_elems);
  const uint8_t *src = in_ptrs[t] + e0 * ES;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const uint32_t nvec = aligned ? n / VE : 0;
  for (int i = tid; i < 256 * COLS; i += HIST_NT) priv[i] = 0;
  __syncthreads();
  auto elem = [](const u32x4 &q, int i) -> uint32_t {
    const int byte = i * ES;
    const uint32_t x = q[byte >> 2];
    if constexpr (ES == 4) return x;
    if constexpr (ES == 2) return (x >> ((byte & 2) * 8)) & 0xFFFF;
    return (x >> ((byte & 3) * 8)) & 0xFF;
  };
  constexpr int B = 4;   // 16-byte loads in flight per thread
  for (uint32_t v0 = tid; v0 < nvec; v0 += B * HIST_NT) {
    u32x4 qs[B];
#pragma unroll
    for (int b = 0; b < B; b++)
      if (v0 + b * HIST_NT < nvec) qs[b] = ldg16(src + 16ull * (v0 + b * HIST_NT));
#pragma unroll
    for (int b = 0; b < B; b++) {
      if (v0 + b * HIST_NT >= nvec) break;
#pragma unroll
      for (int i = 0; i < VE; i++) atomicAdd(&priv[sfield<DT, 0>(elem(qs[b], i)) * COLS + col], 1u);
    }
  }
  for (uint32_t i = nvec * VE + tid; i < n; i += HIST_NT) {
    const uint8_t *p = src + uint64_t(i) * ES;
    uint32_t w = p[0];
    if constexpr (ES >= 2) w |= uint32_t(p[1]) << 8;
    if constexpr (ES == 4) w |= (uint32_t(p[2]) << 16) | (uint32_t(p[3]) << 24);
    atomicAdd(&priv[sfield<DT, 0>(w) * COLS + col], 1u);
  }
  __syncthreads();
  for (int i = tid; i < 256; i += HIST_NT) {
    uint32_t s = 0;
    for (int j = 0; j < COLS; j++) s += priv[i * COLS + ((j + i) & (COLS - 1))];
    hist[uint64_t(c) * 256 + i] = s;
  }
}

__global__ void k_keys(const uint32_t *hist, int stride, int A, DevLayout L, unsigned long long *keys) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= L.n_chunks) return;
  const int t = find_tensor(L, c);
  const uint64_t e0 = uint64_t(c - L.t_chunk0[t]) * L.chunk_elems;
  const uint64_t rem = L.t_n[t] - e0;
  const uint64_t n = rem < L.chunk_elems ? rem : L.chunk_elems;
  unsigned long long s = 0;
  for (int i = 0; i < A; i++) s += (unsigned long long)i * hist[uint64_t(c) * stride + i];
  keys[c] = (s << 16) / n;
}

// Pooled histogram of every group.  Workgroup z takes a slice of at most
// kPoolSlice chunks and adds each chunk's histogram to its group's row in
// LDS (thread s owns symbol s, so no two threads share a counter), for up to
// kPoolGroups groups at a time; the rows then go to pooled[g] with one
// atomic add per non-zero counter.  A slice's counts fit 32 bits: it holds
// at most max(36, M / 2048 + 1) chunks and at most 4096, so its elements are
// fewer than 36 * 2^20, or than 1/2048 of the input plus one chunk, or (with
// more than 8M chunks, which device memory bounds to under 36 KiB each) than
// 4096 * 2^16.
constexpr int kPoolGroups = 32;
constexpr uint32_t kPoolSlice = 4096;
__global__ __launch_bounds__(256) void k_pool(const uint32_t *hist, int stride, int A, uint32_t M,
                                              const uint8_t *map, int K, unsigned long long *pooled) {
  __shared__ uint32_t acc[kPoolGroups][256];
  __shared__ uint8_t gm[kPoolSlice];   // the slice's groups, read once
  const int tid = threadIdx.x;
  const uint32_t per = (M + gridDim.x - 1) / gridDim.x;
  const uint32_t c0 = blockIdx.x * per, c1 = c0 + per < M ? c0 + per : M;
  const uint32_t nc = c1 > c0 ? c1 - c0 : 0u;
  for (uint32_t i = tid; i < nc; i += 256) gm[i] = uint8_t(ldg1(map + c0 + i));
  const uint32_t *hp = hist + uint64_t(c0) * uint32_t(stride) + tid;
  for (int gb = 0; gb < K; gb += kPoolGroups) {
    for (int g = 0; g < kPoolGroups; g++) acc[g][tid] = 0;
    __syncthreads();
    // eight rows in flight at a time; a row's group is the same for every
    // thread
    uint32_t i = 0;
    for (; i + 8 <= nc; i += 8) {
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; j++) h[j] = tid < A ? ldg4(hp + uint64_t(i + j) * uint32_t(stride)) : 0u;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int g = int(gm[i + j]) - gb;
        if (g >= 0 && g < kPoolGroups) acc[g][tid] += h[j];
      }
    }
    for (; i < nc; i++) {
      const int g = int(gm[i]) - gb;
      if (g >= 0 && g < kPoolGroups && tid < A) acc[g][tid] += ldg4(hp + uint64_t(i) * uint32_t(stride));
    }
    __syncthreads();
    for (int g = 0; g < kPoolGroups && gb + g < K; g++)
      if (tid < A && acc[g][tid]) atomicAdd(&pooled[(gb + g) * 256 + tid], (unsigned long long)acc[g][tid]);
    __syncthreads();
  }
}

// One histogram per workgroup: the one-wave package-merge when at most 64
// symbols are present, the workgroup version otherwise (same result).
__global__ __launch_bounds__(256) void k_lengths(const uint64_t *hw, int A, int group_rule,
                                                 uint8_t *len) {
  __shared__ PMShared pm;
  __shared__ WaveCB wcb;
  __shared__ uint64_t w[256];
  __shared__ uint8_t l[256];
  __shared__ int big;
  const int tid = threadIdx.x, h = blockIdx.x;
  w[tid] = tid < A ? hw[uint64_t(h) * 256 + tid] : 0;
  __syncthreads();
  if (tid < 64) {
    const int d = wave_pm_lengths<uint64_t>(w, A, group_rule != 0, l, wcb);
    if (tid == 0) big = d < 0;
  }
  __syncthreads();
  if (big) pm_lengths<256>(pm, w, A, group_rule != 0, l);
  __syncthreads();
  len[uint64_t(h) * 256 + tid] = tid < A ? l[tid] : 0;
}

__global__ __launch_bounds__(256) void k_group_tables(const uint8_t *len, int A, uint32_t *enc,
                                                      uint32_t *lut, uint32_t *ctl) {
  __shared__ uint8_t l[256];
  __shared__ uint32_t e[256];
  __shared__ int cnt[4][kMaxLen + 1];
  __shared__ uint16_t t1[kLutSize];
  __shared__ uint32_t lt[kLutSize];
  __shared__ LutShared ls;
  __shared__ int any;
  const int tid = threadIdx.x, g = blockIdx.x;
  l[tid] = tid < A ? len[g * 256 + tid] : 0;
  if (tid == 0) any = 0;
  __syncthreads();
  if (l[tid]) any = 1;
  __syncthreads();
  if (!any) {  // an empty group: no chunk refers to it
    enc[g * 256 + tid] = 0;
    for (int i = tid; i < kLutSize; i += 256) lut[uint64_t(g) * kLutSize + i] = 0;
    return;
  }
  canon_encode_table(l, A, e, cnt);
  enc[g * 256 + tid] = tid < A ? e[tid] : 0;
  if (!build_lut<256>(l, A, lt, t1, ls)) {
    if (tid == 0) atomicOr(ctl, kErrTableset);
    return;
  }
  for (int i = tid; i < kLutSize; i += 256) lut[uint64_t(g) * kLutSize + i] = lt[i];
}

// Each chunk to the group code of least coded size (ties to the smaller id;
// a chunk that every code lacks a symbol for keeps its group), and cost[0] +=
// its coded size under its current group (all ones if that code lacks one of
// its symbols).  One lane per chunk: for 16 groups at a time the lane sums
// h[s] * len_g[s] over the symbols, the 16 lengths at symbol s being one
// 16-byte LDS read that every lane shares (symbol-major table), so a term
// costs a byte extract and a multiply-add and no lane exchange is needed.
// The sums fit 32 bits (a chunk holds at most 2^20 elements, a length is at
// most 11).  A code lacks one of the chunk's symbols when the chunk's
// present-symbol mask meets the complement of the code's mask.
__device__ __forceinline__ unsigned long long shx64(unsigned long long v, int m) {
  const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(v)), m, 64));
  const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(v >> 32)), m, 64));
  return lo | (uint64_t(hi) << 32);
}
__global__ __launch_bounds__(256) void k_assign(const uint32_t *hist, int stride, int A, uint32_t M,
                                                const uint8_t *len, int K, int reassign, uint8_t *map,
                                                unsigned long long *cost) {
  __shared__ alignas(16) uint8_t lb[256][16];   // lengths of 16 groups at each symbol
  __shared__ uint32_t cmask[16][8];             // bit s: symbol s has a code word
  __shared__ unsigned long long wsum[4];
  const int tid = threadIdx.x, ln = tid & 63;
  const uint32_t c = blockIdx.x * 256u + uint32_t(tid);
  const bool live = c < M;
  const uint32_t *hc = hist + uint64_t(live ? c : 0u) * uint32_t(stride);
  const int cur = live ? int(ldg1(map + c)) : 0;
  uint32_t pres[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // symbols present in the chunk
  unsigned long long best = ~0ull, here = ~0ull;
  int bg = cur;
  auto block16 = [&](int s0, uint32_t (&h)[16]) {   // counts of symbols [s0, s0 + 16)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const u32x4 v = live ? ldg16(hc + s0 + 4 * q) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; j++) h[4 * q + j] = v[j];
    }
  };
  for (int gb = 0; gb < K; gb += 16) {
    __syncthreads();   // the previous batch's tables are no longer read
    for (int i = tid; i < 256 * 16; i += 256) {
      const int sy = i >> 4, g = gb + (i & 15);
      lb[sy][i & 15] = g < K && sy < A ? len[g * 256 + sy] : 0;
    }
    if (tid < 128) {
      const int g = gb + (tid >> 3), w = tid & 7;
      uint32_t m = 0;
      if (g < K)
        for (int j = 0; j < 32; j++) m |= uint32_t(32 * w + j < A && len[g * 256 + 32 * w + j] != 0) << j;
      cmask[tid >> 3][w] = m;
    }
    __syncthreads();
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 16; i++) x[i] = 0;
    // counts loaded one block of 16 symbols ahead
    uint32_t hn[16];
    block16(0, hn);
    for (int s0 = 0; s0 < A; s0 += 16) {
      uint32_t h[16];
#pragma unroll
      for (int j = 0; j < 16; j++) h[j] = hn[j];
      if (s0 + 16 < A) block16(s0 + 16, hn);
      if (gb == 0) {
        uint32_t pm = 0;
#pragma unroll
        for (int j = 0; j < 16; j++) pm |= uint32_t(h[j] != 0) << j;
        pres[s0 >> 5] |= pm << (s0 & 16);
      }
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const uint4 lq = *reinterpret_cast<const uint4 *>(&lb[s0 + j][0]);
        const uint32_t lw[4] = {lq.x, lq.y, lq.z, lq.w};
#pragma unroll
        for (int i = 0; i < 16; i++) x[i] += h[j] * ((lw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (gb + i >= K) break;
      uint32_t miss = 0;
#pragma unroll
      for (int w = 0; w < 8; w++) miss |= pres[w] & ~cmask[i][w];
      const unsigned long long tot = miss ? ~0ull : uint64_t(x[i]);
      if (gb + i == cur) here = tot;
      if (tot < best) {
        best = tot;
        bg = gb + i;
      }
    }
  }
  if (live && reassign) map[c] = uint8_t(bg);
  // modulo 2^64, as one atomic add per chunk would be; one atomic per
  // workgroup, since a single counter taking one add per chunk serialises
  // tens of thousands of them
  unsigned long long v = live ? here : 0ull;
  for (int m = 32; m >= 1; m >>= 1) v += shx64(v, m);
  if (ln == 0) wsum[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) atomicAdd(cost, wsum[0] + wsum[1] + wsum[2] + wsum[3]);
}

// ------------------------------------------------ packed exponent pairs ----
// F of group g: the values of largest pooled count (ties to the smaller
// value), at most 16, present values only; rank[g][v] = v's place in F or
// 0xFF.  One workgroup per group.
__global__ __launch_bounds__(256) void k_pair_F(const unsigned long long *pooled, uint8_t *F, uint8_t *nF,
                                                uint8_t *rank) {
  __shared__ unsigned long long h[256];
  const int tid = threadIdx.x, g = blockIdx.x;
  const unsigned long long mine = pooled[uint64_t(g) * 256 + tid];
  h[tid] = mine;
  __syncthreads();
  int r = 0;   // values ahead of this one in (count descending, value ascending) order
  for (int s = 0; s < 256; s++) {
    const unsigned long long o = h[s];
    r += (o > mine) || (o == mine && s < tid);
  }
  const int present = __syncthreads_count(mine != 0);
  const int n = present < 16 ? present : 16;
  const bool in = mine != 0 && r < 16;
  rank[uint64_t(g) * 256 + tid] = in ? uint8_t(r) : uint8_t(0xFF);
  if (in) F[g * 16 + r] = uint8_t(tid);
  if (tid >= n && tid < 16) F[g * 16 + tid] = 0;
  if (tid == 0) nF[g] = uint8_t(n);
}

// Token counts of the groups: one workgroup per chunk, LDS bins in 4 lane
// columns, then one global add per non-zero bin.  Token 256 + 16 rank(x) +
// rank(y) for an aligned pair of values of F (a 16-byte vector holds 4
// aligned pairs), the single token of each other value.
__global__ __launch_bounds__(256) void k_pair_tokens(DevLayout L, const uint8_t *const *in_ptrs,
                                                     const uint8_t *map, const uint8_t *rank,
                                                     unsigned long long *tok) {
  __shared__ uint32_t bins[4][512];
  __shared__ uint8_t rk[256];
  const int tid = threadIdx.x, col = tid & 3;
  const uint32_t c = blockIdx.x;
  const int g = ldg1(map + c);
  rk[tid] = ldg1(rank + uint64_t(g) * 256 + tid);
  for (int i = tid; i < 4 * 512; i += 256) bins[i >> 9][i & 511] = 0;
  __syncthreads();
  const int t = find_tensor(L, c);
  const uint64_t e0 = uint64_t(c - L.t_chunk0[t]) * L.chunk_elems;
  const uint64_t rem = L.t_n[t] - e0;
  const uint32_t n = uint32_t(rem < L.chunk_elems ? rem : L.chunk_elems);
  const uint8_t *src = in_ptrs[t] + e0 * 2;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const uint32_t nvec = aligned ? n / 8 : 0;
  auto pair = [&](uint32_t x, uint32_t y) {
    const uint32_t rx = rk[x], ry = rk[y];
    if ((rx | ry) < 16) {
      atomicAdd(&bins[col][256 + 16 * rx + ry], 1u);
    } else {
      atomicAdd(&bins[col][x], 1u);
      atomicAdd(&bins[col][y], 1u);
    }
  };
  for (uint32_t v = tid; v < nvec; v += 256) {
    const u32x4 q = ldg16(src + 16ull * v);
#pragma unroll
    for (int i = 0; i < 4; i++) pair((q[i] >> 7) & 0xFF, (q[i] >> 23) & 0xFF);
  }
  for (uint32_t i = nvec * 8 + 2 * tid; i < n; i += 512) {   // the tail, pairs from even positions
    const uint32_t x = (ldg2(src + 2ull * i) >> 7) & 0xFF;
    if (i + 1 < n) pair(x, (ldg2(src + 2ull * i + 2) >> 7) & 0xFF);
    else atomicAdd(&bins[col][x], 1u);   // a lone last value
  }
  __syncthreads();
  for (int i = tid; i < 512; i += 256) {
    const uint32_t v = bins[0][i] + bins[1][i] + bins[2][i] + bins[3][i];
    if (v) atomicAdd(tok + uint64_t(g) * 512 + i, (unsigned long long)v);
  }
}

// Lengths over a group's 512 token counts (the group rule for one token).
__global__ __launch_bounds__(512) void k_token_lengths(const unsigned long long *tok, uint8_t *tlen) {
  __shared__ PMSharedA<512> pm;
  __shared__ uint64_t w[512];
  __shared__ uint8_t l[512];
  const int tid = threadIdx.x, g = blockIdx.x;
  w[tid] = tok[uint64_t(g) * 512 + tid];
  __syncthreads();
  pm_lengths<512, 512>(pm, w, 512, true, l);
  __syncthreads();
  tlen[uint64_t(g) * 512 + tid] = l[tid];
}

// A group packs when its pooled token bits are fewer than its pooled single
// bits under its single-value code.
__global__ __launch_bounds__(256) void k_pair_decide(const unsigned long long *tok, const uint8_t *tlen,
                                                     const unsigned long long *pooled, const uint8_t *len,
                                                     uint8_t *packed) {
  __shared__ unsigned long long sb[4], ss[4];
  const int tid = threadIdx.x, g = blockIdx.x;
  const uint64_t o = uint64_t(g) * 512;
  unsigned long long bt = tok[o + tid] * tlen[o + tid] + tok[o + 256 + tid] * tlen[o + 256 + tid];
  unsigned long long bs = pooled[uint64_t(g) * 256 + tid] * len[uint64_t(g) * 256 + tid];
  bt = wave_sum64(bt);
  bs = wave_sum64(bs);
  if ((tid & 63) == 0) {
    sb[tid >> 6] = bt;
    ss[tid >> 6] = bs;
  }
  __syncthreads();
  if (tid == 0) packed[g] = (sb[0] + sb[1] + sb[2] + sb[3]) < (ss[0] + ss[1] + ss[2] + ss[3]) ? 1 : 0;
}

// Tables of a packing group: canonical codes over the 512 tokens (singles
// into enc and the single lengths into len, pairs into penc), and the decode
// table with one token per entry: the window's bits used | values (1 or 2)
// << 6 | the values, first in bits 8..15.  A token code that is not complete
// is a tableset error.  One workgroup of 512 per group.
__global__ __launch_bounds__(512) void k_pair_tables(const uint8_t *tlen, const uint8_t *F, const uint8_t *packed,
                                                     uint8_t *len, uint32_t *enc, uint32_t *penc, uint32_t *lut,
                                                     uint32_t *ctl) {
  __shared__ int cnt[8][kMaxLen + 1];
  __shared__ uint32_t lt[kLutSize];
  __shared__ uint8_t f[16];
  const int tid = threadIdx.x, g = blockIdx.x, wv = tid >> 6, ln = tid & 63;
  if (!packed[g]) return;
  const int l = tlen[uint64_t(g) * 512 + tid];
  if (tid < 16) f[tid] = F[g * 16 + tid];
  for (int i = tid; i < kLutSize; i += 512) lt[i] = 0;
  int rank = 0;
  for (int b = 1; b <= kMaxLen; b++) {
    const uint64_t m = __ballot(l == b);
    if (l == b) rank = __popcll(m & lanemask_lt());
    if (ln == 0) cnt[wv][b] = __popcll(m);
  }
  const int kr = __syncthreads_count(l != 0) >= 2;
  int kraft_part = l ? 1 << (kMaxLen - l) : 0;
  const int full = kr ? 1 : 0;
  uint32_t e = 0;
  if (l) {
    uint32_t code = 0;
    for (int b = 1; b <= l; b++) {
      int prevc = 0;
      if (b > 1)
        for (int q = 0; q < 8; q++) prevc += cnt[q][b - 1];
      code = (code + prevc) << 1;
    }
    for (int q = 0; q < wv; q++) code += cnt[q][l];
    code += rank;
    e = (__builtin_bitreverse32(code) >> (32 - l)) | (uint32_t(l) << 16);
  }
  if (tid < 256) {
    enc[g * 256 + tid] = e;
    len[g * 256 + tid] = uint8_t(l);
  } else {
    penc[g * 256 + tid - 256] = e;
  }
  // Kraft equality over the tokens
  __shared__ int ksum;
  if (tid == 0) ksum = 0;
  __syncthreads();
  kraft_part = wave_sum(kraft_part);
  if (ln == 0) atomicAdd(&ksum, kraft_part);
  __syncthreads();
  if (!full || ksum != kLutSize) {
    if (tid == 0) atomicOr(ctl, kErrTableset);
    return;
  }
  if (l) {
    const uint32_t vals = tid < 256 ? uint32_t(tid) : uint32_t(f[(tid - 256) >> 4]) | (uint32_t(f[(tid - 256) & 15]) << 8);
    const uint32_t ent = uint32_t(l) | ((tid < 256 ? 1u : 2u) << 6) | (vals << 8);
    const uint32_t rev = e & 0xFFFFu;
    for (uint32_t k = 0; k < (1u << (kMaxLen - l)); k++) lt[rev | (k << l)] = ent;
  }
  __syncthreads();
  for (int i = tid; i < kLutSize; i += 512) lut[uint64_t(g) * kLutSize + i] = lt[i];
}

hipError_t launch_pairs(const DevLayout &L, const uint8_t *const *in_ptrs, const uint8_t *map,
                        const unsigned long long *pooled, const uint8_t *len, int K, uint8_t *F, uint8_t *nF,
                        uint8_t *rank, unsigned long long *tok, uint8_t *tlen, uint8_t *packed, hipStream_t s) {
  if (K <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pair_F, dim3(K), dim3(256), 0, s, pooled, F, nF, rank);
  if (L.n_chunks) hipLaunchKernelGGL(k_pair_tokens, dim3(L.n_chunks), dim3(256), 0, s, L, in_ptrs, map, rank, tok);
  hipLaunchKernelGGL(k_token_lengths, dim3(K), dim3(512), 0, s, tok, tlen);
  hipLaunchKernelGGL(k_pair_decide, dim3(K), dim3(256), 0, s, tok, tlen, pooled, len, packed);
  return hipGetLastError();
}

hipError_t launch_pair_tables(const uint8_t *tlen, const uint8_t *F, const uint8_t *packed, int K, uint8_t *len,
                              uint32_t *enc, uint32_t *penc, uint32_t *lut, uint32_t *ctl, hipStream_t s) {
  if (K <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pair_tables, dim3(K), dim3(512), 0, s, tlen, F, packed, len, enc, penc, lut, ctl);
  return hipGetLastError();
}

hipError_t launch_hist_all(int dtype, const DevLayout &L, const uint8_t *const *in_ptrs,
                           uint32_t *hist, hipStream_t s) {
  if (!L.n_chunks) return hipSuccess;
  const dim3 grid(L.n_chunks), block(HIST_NT);
  if (dtype == BF16) hipLaunchKernelGGL(k_hist_all<BF16>, grid, block, 0, s, L, in_ptrs, hist);
  else if (dtype == FP32) hipLaunchKernelGGL(k_hist_all<FP32>, grid, block, 0, s, L, in_ptrs, hist);
  else if (dtype == FP8) hipLaunchKernelGGL(k_hist_all<FP8>, grid, block, 0, s, L, in_ptrs, hist);
  else hipLaunchKernelGGL(k_hist_all<FP4X2>, grid, block, 0, s, L, in_ptrs, hist);
  return hipGetLastError();
}

hipError_t launch_hist0(int dtype, const DevLayout &L, const uint8_t *const *in_ptrs, uint32_t *hist,
                        hipStream_t s) {
  if (!L.n_chunks) return hipSuccess;
  const dim3 grid(L.n_chunks), block(HIST_NT);
  if (dtype == BF16) hipLaunchKernelGGL(k_hist0<BF16>, grid, block, 0, s, L, in_ptrs, hist);
  else if (dtype == FP32) hipLaunchKernelGGL(k_hist0<FP32>, grid, block, 0, s, L, in_ptrs, hist);
  else if (dtype == FP8) hipLaunchKernelGGL(k_hist0<FP8>, grid, block, 0, s, L, in_ptrs, hist);
  else hipLaunchKernelGGL(k_hist0<FP4X2>, grid, block, 0, s, L, in_ptrs, hist);
  return hipGetLastError();
}

hipError_t launch_keys(const uint32_t *hist, int stride, int A, const DevLayout &L,
                       unsigned long long *keys, hipStream_t s) {
  if (!L.n_chunks) return hipSuccess;
  hipLaunchKernelGGL(k_keys, dim3((L.n_chunks + 255) / 256), dim3(256), 0, s, hist, stride, A, L, keys);
  return hipGetLastError();
}

hipError_t launch_pool(const uint32_t *hist, int stride, int A, uint32_t M, const uint8_t *map,
                       unsigned long long *pooled, int K, hipStream_t s) {
  if (!M || K <= 0) return hipSuccess;
  // about 36 chunks per workgroup, at most kPoolSlice
  uint32_t slices = (M + 35) / 36;
  if (slices > 2048) slices = 2048;
  if ((M + slices - 1) / slices > kPoolSlice) slices = (M + kPoolSlice - 1) / kPoolSlice;
  hipLaunchKernelGGL(k_pool, dim3(slices), dim3(256), 0, s, hist, stride, A, M, map, K, pooled);
  return hipGetLastError();
}

hipError_t launch_lengths(const uint64_t *hw, int n, int A, int group_rule, uint8_t *len,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lengths, dim3(n), dim3(256), 0, s, hw, A, group_rule, len);
  return hipGetLastError();
}

hipError_t launch_group_tables(const uint8_t *len, int K, int A, uint32_t *enc, uint32_t *lut,
                               uint32_t *ctl, hipStream_t s) {
  if (K <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_group_tables, dim3(K), dim3(256), 0, s, len, A, enc, lut, ctl);
  return hipGetLastError();
}

hipError_t launch_assign(const uint32_t *hist, int stride, int A, uint32_t M, const uint8_t *len,
                         int K, int reassign, uint8_t *map, unsigned long long *cost, hipStream_t s) {
  if (!M || K <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_assign, dim3((M + 255) / 256), dim3(256), 0, s, hist, stride, A, M, len, K, reassign,
                     map, cost);
  return hipGetLastError();
}

}  // namespace zn
