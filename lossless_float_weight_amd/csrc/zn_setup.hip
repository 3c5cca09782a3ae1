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
// atomic add per non-zero counter.  A slice's counts fit 32 bits: at most
// 4096 chunks of at most 2^19 elements.
constexpr int kPoolGroups = 32;
constexpr uint32_t kPoolSlice = 4096;
__global__ __launch_bounds__(256) void k_pool(const uint32_t *hist, int stride, int A, uint32_t M,
                                              const uint8_t *map, int K, unsigned long long *pooled) {
  __shared__ uint32_t acc[kPoolGroups][256];
  const int tid = threadIdx.x;
  const uint32_t per = (M + gridDim.x - 1) / gridDim.x;
  const uint32_t c0 = blockIdx.x * per, c1 = c0 + per < M ? c0 + per : M;
  for (int gb = 0; gb < K; gb += kPoolGroups) {
    for (int g = 0; g < kPoolGroups; g++) acc[g][tid] = 0;
    __syncthreads();
    for (uint32_t c = c0; c < c1; c++) {
      const int g = int(ldg1(map + c)) - gb;   // the same for every thread
      if (g >= 0 && g < kPoolGroups && tid < A) acc[g][tid] += ldg4(hist + uint64_t(c) * stride + tid);
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
// its symbols).  The K code-length tables wait in LDS; one wave per chunk at a
// time.  Lane l holds the counts of symbols l, l+64, l+128, l+192; for 16
// groups at once it forms the partial sums sum_s h[s]*len_g[s], plus 2^40 per
// present symbol without a code word (every true sum is below 2^40), and a
// butterfly over the lanes halves the set of groups a lane carries at each
// of its first four steps (17 exchanges instead of 16 full reductions):
// afterwards lane l holds the total of group 8*b5 + 4*b4 + 2*b3 + b2, bi the
// bits of l.
constexpr unsigned long long kMissUnit = 1ull << 40;
__device__ __forceinline__ unsigned long long shx64(unsigned long long v, int m) {
  const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(v)), m, 64));
  const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(v >> 32)), m, 64));
  return lo | (uint64_t(hi) << 32);
}
__global__ __launch_bounds__(256) void k_assign(const uint32_t *hist, int stride, int A, uint32_t M,
                                                const uint8_t *len, int K, int reassign, uint8_t *map,
                                                unsigned long long *cost) {
  extern __shared__ uint8_t lsh[];   // [K][256] code lengths
  const int tid = threadIdx.x, ln = tid & 63;
  for (int i = tid; i < K * 256; i += 256) lsh[i] = len[i];
  __syncthreads();
  const uint32_t nw = gridDim.x * 4;
  unsigned long long wave_cost = 0;   // this wave's chunks, added to cost[0] once per workgroup
  for (uint32_t c = blockIdx.x * 4 + (tid >> 6); c < M; c += nw) {
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int s = ln + 64 * q;
      h[q] = s < A ? ldg4(hist + uint64_t(c) * stride + s) : 0u;
    }
    const int cur = ldg1(map + c);
    unsigned long long best = ~0ull, here = ~0ull;
    int bg = cur;
    for (int gb = 0; gb < K; gb += 16) {
      unsigned long long v[16];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int g = gb + i;
        unsigned long long x = 0;
        if (g < K) {
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int s = ln + 64 * q;
            const uint32_t l = s < A ? lsh[g * 256 + s] : 0u;
            x += uint64_t(h[q]) * l + (h[q] && !l ? kMissUnit : 0ull);
          }
        }
        v[i] = x;
      }
#pragma unroll
      for (int half = 8, m = 32; half >= 1; half >>= 1, m >>= 1) {
        const bool up = (ln & m) != 0;
#pragma unroll
        for (int i = 0; i < half; i++) {
          const unsigned long long keep = up ? v[half + i] : v[i];
          const unsigned long long send = up ? v[i] : v[half + i];
          v[i] = keep + shx64(send, m);
        }
      }
      unsigned long long t = v[0];
      t += shx64(t, 2);
      t += shx64(t, 1);
      // group gb + i is in the lanes whose bits 5..2 are i's bits 3..0
#pragma unroll
      for (int i = 0; i < 16 && gb + i < K; i++) {
        const int lane = ((i & 8) ? 32 : 0) | ((i & 4) ? 16 : 0) | ((i & 2) ? 8 : 0) | ((i & 1) ? 4 : 0);
        const unsigned long long tot = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(t >> 32)), lane))) << 32) |
                                       uint32_t(__builtin_amdgcn_readlane(int(uint32_t(t)), lane));
        const unsigned long long x = tot >= kMissUnit ? ~0ull : tot;
        if (gb + i == cur) here = x;
        if (x < best) {
          best = x;
          bg = gb + i;
        }
      }
    }
    if (ln == 0 && reassign) map[c] = uint8_t(bg);
    wave_cost += here;   // modulo 2^64, as one atomic add per chunk would be
  }
  // one atomic per workgroup: a single counter taking one add per chunk
  // serialises tens of thousands of them
  __shared__ unsigned long long wsum[4];
  if (ln == 0) wsum[tid >> 6] = wave_cost;
  __syncthreads();
  if (tid == 0) atomicAdd(cost, wsum[0] + wsum[1] + wsum[2] + wsum[3]);
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
  const uint32_t blocks = (M + 3) / 4 < 2048 ? (M + 3) / 4 : 2048;
  hipLaunchKernelGGL(k_assign, dim3(blocks), dim3(256), size_t(K) * 256, s, hist, stride, A, M, len, K,
                     reassign, map, cost);
  return hipGetLastError();
}

}  // namespace zn
