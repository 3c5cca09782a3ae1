// zn_setup.hip -- kernels of the reusable setup ("NeuralZip: Reusable Setup
// for Fast Lossless Compression", Abstract: chunks with similar exponent
// distributions are grouped and share one Huffman code, chosen once before
// later encodings).  All arithmetic is integer, so the grouping equals the
// CPU oracle's exactly:
//   k_hist_all     order-0 histograms of every coded stream of every chunk
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

// grid (K, slices): workgroup (g, z) sums the histograms of group g's chunks
// in slice z, then adds them to pooled[g].
__global__ __launch_bounds__(256) void k_pool(const uint32_t *hist, int stride, int A, uint32_t M,
                                              const uint8_t *map, unsigned long long *pooled) {
  const int g = blockIdx.x, tid = threadIdx.x;
  const uint32_t per = (M + gridDim.y - 1) / gridDim.y;
  const uint32_t c0 = blockIdx.y * per, c1 = c0 + per < M ? c0 + per : M;
  unsigned long long acc = 0;
  for (uint32_t c = c0; c < c1; c++)
    if (map[c] == g && tid < A) acc += hist[uint64_t(c) * stride + tid];
  if (tid < A && acc) atomicAdd(&pooled[g * 256 + tid], acc);
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

// One wave per chunk: cost under every group code, then the cheapest group
// (ties to the smaller id).  cost[0] += cost under the current assignment.
__global__ __launch_bounds__(256) void k_assign(const uint32_t *hist, int stride, int A, uint32_t M,
                                                const uint8_t *len, int K, int reassign, uint8_t *map,
                                                unsigned long long *cost) {
  const int ln = threadIdx.x & 63;
  const uint32_t c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= M) return;
  uint32_t h[4];
  for (int q = 0; q < 4; q++) {
    const int s = ln + 64 * q;
    h[q] = s < A ? hist[uint64_t(c) * stride + s] : 0;
  }
  const int cur = map[c];
  unsigned long long best = ~0ull, here = 0;
  int bg = cur;
  for (int g = 0; g < K; g++) {
    unsigned long long sum = 0;
    int miss = 0;
    for (int q = 0; q < 4; q++) {
      const int s = ln + 64 * q;
      if (s >= A) continue;
      const uint32_t l = len[g * 256 + s];
      if (h[q] && !l) miss = 1;
      sum += (unsigned long long)h[q] * l;
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    miss = __ballot(miss) != 0;
    const unsigned long long x = miss ? ~0ull : sum;
    if (g == cur) here = x;
    if (x < best) {
      best = x;
      bg = g;
    }
  }
  if (ln == 0) {
    if (reassign) map[c] = uint8_t(bg);
    atomicAdd(cost, here);
  }
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

hipError_t launch_keys(const uint32_t *hist, int stride, int A, const DevLayout &L,
                       unsigned long long *keys, hipStream_t s) {
  if (!L.n_chunks) return hipSuccess;
  hipLaunchKernelGGL(k_keys, dim3((L.n_chunks + 255) / 256), dim3(256), 0, s, hist, stride, A, L, keys);
  return hipGetLastError();
}

hipError_t launch_pool(const uint32_t *hist, int stride, int A, uint32_t M, const uint8_t *map,
                       unsigned long long *pooled, int K, hipStream_t s) {
  const uint32_t slices = M < 64 ? (M ? M : 1) : 64;
  hipLaunchKernelGGL(k_pool, dim3(K, slices), dim3(256), 0, s, hist, stride, A, M, map, pooled);
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
  if (!M) return hipSuccess;
  hipLaunchKernelGGL(k_assign, dim3((M + 3) / 4), dim3(256), 0, s, hist, stride, A, M, len, K, reassign,
                     map, cost);
  return hipGetLastError();
}

}  // namespace zn
