// zn_api.hip -- the C ABI of libzn.so (declared in include/zn.h).
//
// Host code: argument checks, the container layout, the tableset (plan plus
// optional group tables) and the order of launches on the caller's stream.
// Every step of compression and decompression runs in the kernels of
// zn_encode.hip / zn_decode.hip; the setup's only host step is sorting the
// chunk keys once for the initial groups.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/zn.h"
#include "zn_internal.h"

using namespace zn;

// Events that take the start and end times of kernel launches
// (zn_debug_kernel_events); the launches attach them to their dispatches.
namespace {
const char *const kKernelNames[] = {"analyze", "finish", "pack", "check", "decode"};
enum { KAnalyze, KFinish, KPack, KCheck, KDecode, KCount };
hipEvent_t g_ev_before[KCount], g_ev_after[KCount];
}  // namespace

struct zn_tableset {
  int dtype = 0, T = 0, K = 0;
  uint32_t chunk_bytes = 0, chunk_elems = 0, n_chunks = 0;
  uint64_t off_dir = 0, off_records = 0, hash = 0;
  std::vector<uint64_t> n, raw;
  std::vector<uint32_t> chunk0;
  std::vector<uint8_t> hdr;            // header template + tensor table
  std::vector<uint8_t> len;            // [K][256] group code lengths
  std::vector<uint8_t> map;            // [n_chunks] group of each chunk
  std::vector<unsigned long long> cost;  // objective per setup round (diagnostic)
  // packed exponent pairs (pairs = 1 when the setup was asked for them):
  // per group the packing flag, |F|, F[16] and the 512 token lengths
  int pairs = 0;
  std::vector<uint8_t> packed, nF, F, tlen;
  // device copies
  uint64_t *d_n = nullptr, *d_raw = nullptr;
  uint32_t *d_chunk0 = nullptr;
  uint8_t *d_hdr = nullptr;
  uint8_t *d_map = nullptr, *d_len = nullptr;
  uint32_t *d_enc = nullptr, *d_lut = nullptr;
  // for packing groups: len/enc/lut hold the token code's singles and its
  // one-token decode table; penc the pair tokens' codes, rank F's ranks
  uint8_t *d_packed = nullptr, *d_rank = nullptr;
  uint32_t *d_penc = nullptr;
  // the device that was current when the device copies were made: they live
  // there, so every launch with this tableset needs that device current
  int device = -1;
};

namespace {

bool valid_dtype(int dt) { return dt == BF16 || dt == FP32 || dt == FP8 || dt == FP4X2; }
bool valid_chunk(uint32_t cb) { return cb >= 4096 && cb <= (1u << 20) && cb % 4096 == 0; }

void put_u16(uint8_t *p, uint32_t v) { p[0] = v & 0xFF; p[1] = (v >> 8) & 0xFF; }
void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (v >> (8 * i)) & 0xFF; }
void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (v >> (8 * i)) & 0xFF; }
uint32_t get_u16(const uint8_t *p) { return p[0] | (uint32_t(p[1]) << 8); }
uint32_t get_u32(const uint8_t *p) { return p[0] | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16) | (uint32_t(p[3]) << 24); }
uint64_t get_u64(const uint8_t *p) { uint64_t v = 0; for (int i = 7; i >= 0; i--) v = (v << 8) | p[i]; return v; }

#define HIPCHK(x)                        \
  do {                                   \
    if ((x) != hipSuccess) return ZN_ERR_HIP; \
  } while (0)

DevLayout dev_layout(const zn_tableset *ts) {
  DevLayout L;
  L.t_n = ts->d_n;
  L.t_raw = ts->d_raw;
  L.t_chunk0 = ts->d_chunk0;
  L.T = ts->T;
  L.n_chunks = ts->n_chunks;
  L.chunk_elems = ts->chunk_elems;
  L.off_dir = ts->off_dir;
  L.off_records = ts->off_records;
  return L;
}

int alphabet0(int dt) { return 1 << kbits(dt, 0); }

// per group of a version-2 tableset (with pairs): packing flag, |F|, F[16],
// the 512 token lengths two per byte (even token in the low nibble)
constexpr int kTsPairBytes = 274;
uint64_t serial_bytes(const zn_tableset *ts) {
  return 24 + 8ull * ts->T + uint64_t(ts->K) * (alphabet0(ts->dtype) / 2) + ts->n_chunks +
         (ts->pairs ? uint64_t(ts->K) * kTsPairBytes : 0);
}
void serialise(const zn_tableset *ts, uint8_t *b) {
  const int A = alphabet0(ts->dtype);
  put_u32(b, kTsMagic);
  put_u16(b + 4, ts->pairs ? 2 : kVersion);
  b[6] = uint8_t(ts->dtype);
  b[7] = uint8_t(ts->K);
  put_u32(b + 8, ts->chunk_bytes);
  put_u32(b + 12, uint32_t(ts->T));
  put_u32(b + 16, ts->n_chunks);
  put_u32(b + 20, kMaxLen);
  uint8_t *q = b + 24;
  for (int t = 0; t < ts->T; t++, q += 8) put_u64(q, ts->n[t]);
  for (int g = 0; g < ts->K; g++)
    for (int s = 0; s < A; s += 2) *q++ = uint8_t(ts->len[g * 256 + s] | (ts->len[g * 256 + s + 1] << 4));
  if (ts->n_chunks) memcpy(q, ts->map.data(), ts->n_chunks);
  q += ts->n_chunks;
  for (int g = 0; ts->pairs && g < ts->K; g++) {
    *q++ = ts->packed[g];
    *q++ = ts->nF[g];
    memcpy(q, ts->F.data() + 16 * g, 16);
    q += 16;
    for (int t = 0; t < 512; t += 2) *q++ = uint8_t(ts->tlen[512 * g + t] | (ts->tlen[512 * g + t + 1] << 4));
  }
}
uint64_t fnv1a64(const uint8_t *b, uint64_t n) {
  uint64_t h = 14695981039346656037ull;
  for (uint64_t i = 0; i < n; i++) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

// The current device is the tableset's own (a tableset that never reached
// its device copies has none, and every call that launches refuses it).
bool on_device(const zn_tableset *ts) {
  int dev = -1;
  return ts->device >= 0 && hipGetDevice(&dev) == hipSuccess && dev == ts->device;
}

// Frees on the device that holds the memory, then makes the caller's device
// current again.
void free_device(zn_tableset *ts) {
  int cur = -1;
  const bool sw = ts->device >= 0 && hipGetDevice(&cur) == hipSuccess && cur != ts->device &&
                  hipSetDevice(ts->device) == hipSuccess;
  (void)hipFree(ts->d_n);
  (void)hipFree(ts->d_raw);
  (void)hipFree(ts->d_chunk0);
  (void)hipFree(ts->d_hdr);
  (void)hipFree(ts->d_map);
  (void)hipFree(ts->d_len);
  (void)hipFree(ts->d_enc);
  (void)hipFree(ts->d_lut);
  (void)hipFree(ts->d_packed);
  (void)hipFree(ts->d_rank);
  (void)hipFree(ts->d_penc);
  ts->d_n = ts->d_raw = nullptr;
  ts->d_chunk0 = nullptr;
  ts->d_hdr = ts->d_map = ts->d_len = nullptr;
  ts->d_enc = ts->d_lut = nullptr;
  ts->d_packed = ts->d_rank = nullptr;
  ts->d_penc = nullptr;
  if (sw) (void)hipSetDevice(cur);
}

// Host layout of the container for the plan's tensors.
zn_status make_plan(zn_tableset *ts, int dt, const uint64_t *n, int T, uint32_t cb) {
  if (!valid_dtype(dt) || !valid_chunk(cb) || T < 1 || !n) return ZN_ERR_ARG;
  ts->dtype = dt;
  ts->T = T;
  ts->chunk_bytes = cb;
  ts->chunk_elems = cb / uint32_t(esize(dt));
  ts->n.assign(n, n + T);
  ts->raw.assign(T, 0);
  ts->chunk0.assign(T + 1, 0);
  uint64_t M = 0;
  for (int t = 0; t < T; t++) {
    if (n[t] > (1ull << 40)) return ZN_ERR_ARG;
    ts->chunk0[t] = uint32_t(M);
    M += (n[t] + ts->chunk_elems - 1) / ts->chunk_elems;
    if (M > 0x7FFFFFFFull) return ZN_ERR_ARG;
  }
  ts->chunk0[T] = uint32_t(M);
  ts->n_chunks = uint32_t(M);
  ts->off_dir = 64 + 16ull * T;
  uint64_t cur = align16(ts->off_dir + 8 * (M + 1));
  for (int t = 0; t < T; t++) {
    ts->raw[t] = cur;
    cur = align16(cur + rawplane_bytes(dt, n[t]));
  }
  ts->off_records = cur;
  ts->map.assign(M, 0);
  return ZN_OK;
}

// Header template (total_bytes left 0), hash, and device copies of the plan.
zn_status finish_plan(zn_tableset *ts) {
  std::vector<uint8_t> ser(serial_bytes(ts));
  serialise(ts, ser.data());
  ts->hash = fnv1a64(ser.data(), ser.size());
  uint64_t ntot = 0;
  for (auto v : ts->n) ntot += v;
  ts->hdr.assign(64 + 16ull * ts->T, 0);
  uint8_t *h = ts->hdr.data();
  put_u32(h, kMagic);
  put_u16(h + 4, kVersion);
  h[6] = uint8_t(ts->dtype);
  h[7] = ts->K ? 1 : 0;
  put_u32(h + 8, uint32_t(ts->T));
  put_u32(h + 12, ts->chunk_bytes);
  put_u64(h + 16, ntot);
  put_u32(h + 24, ts->n_chunks);
  put_u16(h + 28, uint32_t(segsyms(ts->dtype)));
  h[30] = kMaxLen;
  h[31] = uint8_t(ncoded(ts->dtype));
  put_u64(h + 32, ts->K ? ts->hash : 0);
  put_u64(h + 40, ts->off_dir);
  put_u64(h + 48, ts->off_records);
  for (int t = 0; t < ts->T; t++) {
    put_u64(h + 64 + 16 * t, ts->n[t]);
    put_u64(h + 72 + 16 * t, ts->raw[t]);
  }
  if (!ts->d_n) {
    HIPCHK(hipGetDevice(&ts->device));
    HIPCHK(hipMalloc(&ts->d_n, 8ull * ts->T));
    HIPCHK(hipMalloc(&ts->d_raw, 8ull * ts->T));
    HIPCHK(hipMalloc(&ts->d_chunk0, 4ull * (ts->T + 1)));
    HIPCHK(hipMalloc(&ts->d_hdr, ts->hdr.size()));
  }
  HIPCHK(hipMemcpy(ts->d_n, ts->n.data(), 8ull * ts->T, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(ts->d_raw, ts->raw.data(), 8ull * ts->T, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(ts->d_chunk0, ts->chunk0.data(), 4ull * (ts->T + 1), hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(ts->d_hdr, ts->hdr.data(), ts->hdr.size(), hipMemcpyHostToDevice));
  return ZN_OK;
}

struct DevBufU8 {
  uint8_t *p = nullptr;
  ~DevBufU8() { (void)hipFree(p); }
  hipError_t alloc(size_t n) { return hipMalloc(&p, n ? n : 1); }
};

// Device group tables (encode codes, decode tables) from host lengths and map.
zn_status upload_groups(zn_tableset *ts, hipStream_t s) {
  const int K = ts->K;
  if (!K) return ZN_OK;
  if (!ts->d_map) {
    HIPCHK(hipMalloc(&ts->d_map, ts->n_chunks ? ts->n_chunks : 1));
    HIPCHK(hipMalloc(&ts->d_len, 256ull * K));
    HIPCHK(hipMalloc(&ts->d_enc, 4ull * 256 * K));
    HIPCHK(hipMalloc(&ts->d_lut, 4ull * kLutSize * K));
  }
  if (ts->n_chunks)
    HIPCHK(hipMemcpyAsync(ts->d_map, ts->map.data(), ts->n_chunks, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(ts->d_len, ts->len.data(), 256ull * K, hipMemcpyHostToDevice, s));
  // packing flags (all zero without pairs) and F's ranks, for the kernels
  std::vector<uint8_t> pk(K, 0), rank(256ull * K, 0xFF);
  for (int g = 0; ts->pairs && g < K; g++) {
    pk[g] = ts->packed[g];
    for (int i = 0; i < ts->nF[g]; i++) rank[256ull * g + ts->F[16 * g + i]] = uint8_t(i);
  }
  if (!ts->d_packed) {
    HIPCHK(hipMalloc(&ts->d_packed, K));
    HIPCHK(hipMalloc(&ts->d_rank, 256ull * K));
    HIPCHK(hipMalloc(&ts->d_penc, 4ull * 256 * K));
  }
  HIPCHK(hipMemcpyAsync(ts->d_packed, pk.data(), K, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(ts->d_rank, rank.data(), 256ull * K, hipMemcpyHostToDevice, s));
  DevBufU8 tl, fv;
  uint32_t *ctl = nullptr;
  HIPCHK(hipMalloc(&ctl, 4));
  HIPCHK(hipMemsetAsync(ctl, 0, 4, s));
  hipError_t e = launch_group_tables(ts->d_len, K, alphabet0(ts->dtype), ts->d_enc, ts->d_lut, ctl, s);
  if (e == hipSuccess && ts->pairs) {
    e = tl.alloc(512ull * K);
    if (e == hipSuccess) e = fv.alloc(16ull * K);
    if (e == hipSuccess) e = hipMemcpyAsync(tl.p, ts->tlen.data(), 512ull * K, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(fv.p, ts->F.data(), 16ull * K, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = launch_pair_tables(tl.p, fv.p, ts->d_packed, K, ts->d_len, ts->d_enc, ts->d_penc, ts->d_lut, ctl, s);
  }
  uint32_t flag = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&flag, ctl, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(ctl);
  if (e != hipSuccess) return ZN_ERR_HIP;
  return flag ? ZN_ERR_TABLESET : ZN_OK;
}

template <class T>
struct DevBuf {
  T *p = nullptr;
  ~DevBuf() { (void)hipFree(p); }
  hipError_t alloc(size_t n) { return hipMalloc(&p, sizeof(T) * (n ? n : 1)); }
};

// NeuralZip grouping on the GPU (integer Lloyd rounds); see zn_setup.hip.
zn_status run_grouping(zn_tableset *ts, const void *const *d_tensors, hipStream_t s) {
  const int dt = ts->dtype, K = ts->K, A = alphabet0(dt);
  const uint32_t M = ts->n_chunks;
  const int stride = 256;   // the exponent stream's histogram only
  ts->len.assign(256ull * K, 0);
  ts->cost.assign(kRounds + 1, 0);
  DevBuf<const uint8_t *> ptrs;
  DevBuf<uint32_t> hist;
  DevBuf<unsigned long long> keys, pooled, cost;
  DevBuf<uint8_t> map, len;
  if (ptrs.alloc(ts->T) || hist.alloc(uint64_t(M) * stride) || keys.alloc(M) ||
      pooled.alloc(256ull * K) || cost.alloc(kRounds + 1) || map.alloc(M) || len.alloc(256ull * K))
    return ZN_ERR_NOMEM;
  HIPCHK(hipMemcpyAsync(ptrs.p, d_tensors, sizeof(void *) * ts->T, hipMemcpyHostToDevice, s));
  const DevLayout L = dev_layout(ts);
  HIPCHK(launch_hist0(dt, L, ptrs.p, hist.p, s));
  HIPCHK(launch_keys(hist.p, stride, A, L, keys.p, s));
  std::vector<unsigned long long> hkeys(M);
  HIPCHK(hipMemcpyAsync(hkeys.data(), keys.p, 8ull * M, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  // initial groups: chunks ordered by (key, chunk), cut into K even runs.
  // A key is below 256 * 2^16 = 2^24: three stable counting passes over its
  // bytes (least significant first) starting from chunk order give exactly
  // that order.
  std::vector<uint32_t> order(M), tmp(M);
  for (uint32_t c = 0; c < M; c++) order[c] = c;
  for (int pass = 0; pass < 3; pass++) {
    uint32_t cnt[257] = {0};
    const int sh = 8 * pass;
    for (uint32_t i = 0; i < M; i++) cnt[((hkeys[order[i]] >> sh) & 0xFF) + 1]++;
    for (int b = 0; b < 256; b++) cnt[b + 1] += cnt[b];
    for (uint32_t i = 0; i < M; i++) tmp[cnt[(hkeys[order[i]] >> sh) & 0xFF]++] = order[i];
    order.swap(tmp);
  }
  for (int g = 0; g < K; g++)
    for (uint64_t i = uint64_t(M) * g / K; i < uint64_t(M) * (g + 1) / K; i++) ts->map[order[i]] = uint8_t(g);
  HIPCHK(hipMemcpyAsync(map.p, ts->map.data(), M, hipMemcpyHostToDevice, s));
  // every round's cost goes to its own word, read back once at the end
  HIPCHK(hipMemsetAsync(cost.p, 0, 8ull * (kRounds + 1), s));
  for (int r = 0; r <= kRounds; r++) {
    HIPCHK(hipMemsetAsync(pooled.p, 0, 8 * 256ull * K, s));
    HIPCHK(launch_pool(hist.p, stride, A, M, map.p, pooled.p, K, s));
    HIPCHK(launch_lengths(reinterpret_cast<const uint64_t *>(pooled.p), K, A, 1, len.p, s));
    // the last pass only measures the final assignment
    HIPCHK(launch_assign(hist.p, stride, A, M, len.p, K, r < kRounds, map.p, cost.p + r, s));
  }
  HIPCHK(hipMemcpyAsync(ts->cost.data(), cost.p, 8ull * (kRounds + 1), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(ts->len.data(), len.p, 256ull * K, hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(ts->map.data(), map.p, M, hipMemcpyDeviceToHost, s));
  if (ts->pairs) {
    // packed exponent pairs from the final assignment: pooled holds the final
    // groups' histograms (the last round measures only) and len their codes
    DevBuf<unsigned long long> tok;
    DevBuf<uint8_t> F, nF, rank, tlen, packed;
    if (tok.alloc(512ull * K) || F.alloc(16ull * K) || nF.alloc(K) || rank.alloc(256ull * K) ||
        tlen.alloc(512ull * K) || packed.alloc(K))
      return ZN_ERR_NOMEM;
    HIPCHK(hipMemsetAsync(tok.p, 0, 8 * 512ull * K, s));
    HIPCHK(launch_pairs(L, ptrs.p, map.p, pooled.p, len.p, K, F.p, nF.p, rank.p, tok.p, tlen.p, packed.p, s));
    ts->F.assign(16ull * K, 0);
    ts->nF.assign(K, 0);
    ts->tlen.assign(512ull * K, 0);
    ts->packed.assign(K, 0);
    HIPCHK(hipMemcpyAsync(ts->F.data(), F.p, 16ull * K, hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(ts->nF.data(), nF.p, K, hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(ts->tlen.data(), tlen.p, 512ull * K, hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(ts->packed.data(), packed.p, K, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
  }
  HIPCHK(hipStreamSynchronize(s));
  return ZN_OK;
}

// Content-based assignment of a transferred setup: every chunk of the new
// tensors to the group code of least coded size (ties to the smaller id; a
// chunk that every code lacks a symbol for stays in group 0).
zn_status run_transfer(zn_tableset *ts, const void *const *d_tensors, hipStream_t s) {
  const int dt = ts->dtype, K = ts->K, A = alphabet0(dt);
  const uint32_t M = ts->n_chunks;
  const int stride = 256;   // the exponent stream's histogram only
  DevBuf<const uint8_t *> ptrs;
  DevBuf<uint32_t> hist;
  DevBuf<unsigned long long> cost;
  DevBuf<uint8_t> map, len;
  if (ptrs.alloc(ts->T) || hist.alloc(uint64_t(M) * stride) || cost.alloc(1) || map.alloc(M) ||
      len.alloc(256ull * K))
    return ZN_ERR_NOMEM;
  HIPCHK(hipMemcpyAsync(ptrs.p, d_tensors, sizeof(void *) * ts->T, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(len.p, ts->len.data(), 256ull * K, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemsetAsync(map.p, 0, M ? M : 1, s));
  HIPCHK(hipMemsetAsync(cost.p, 0, 8, s));
  const DevLayout L = dev_layout(ts);
  HIPCHK(launch_hist0(dt, L, ptrs.p, hist.p, s));
  HIPCHK(launch_assign(hist.p, stride, A, M, len.p, K, 1, map.p, cost.p, s));
  if (M) HIPCHK(hipMemcpyAsync(ts->map.data(), map.p, M, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  return ZN_OK;
}

}  // namespace

extern "C" {

const char *zn_status_str(zn_status s) {
  switch (s) {
    case ZN_OK: return "ok";
    case ZN_ERR_ARG: return "invalid argument";
    case ZN_ERR_CORRUPT: return "corrupt container";
    case ZN_ERR_CAPACITY: return "buffer too small";
    case ZN_ERR_TABLESET: return "tableset mismatch";
    case ZN_ERR_HIP: return "HIP runtime error";
    case ZN_ERR_NOMEM: return "out of memory";
  }
  return "unknown status";
}

void zn_tableset_free(zn_tableset *ts) {
  if (!ts) return;
  free_device(ts);
  delete ts;
}

zn_status zn_setup(zn_dtype dtype, const void *const *d_tensors, const uint64_t *n_elems,
                   int n_tensors, uint32_t chunk_bytes, int n_groups, hipStream_t stream,
                   zn_tableset **out) {
  return zn_setup2(dtype, d_tensors, n_elems, n_tensors, chunk_bytes, n_groups, 0, stream, out);
}

zn_status zn_setup2(zn_dtype dtype, const void *const *d_tensors, const uint64_t *n_elems,
                    int n_tensors, uint32_t chunk_bytes, int n_groups, int flags, hipStream_t stream,
                    zn_tableset **out) {
  if (!out || n_groups < 0 || n_groups > 255) return ZN_ERR_ARG;
  *out = nullptr;
  if ((flags & ~ZN_SETUP_PAIRS) || ((flags & ZN_SETUP_PAIRS) && (dtype != ZN_BF16 || n_groups < 1)))
    return ZN_ERR_ARG;
  zn_tableset *ts = new (std::nothrow) zn_tableset;
  if (!ts) return ZN_ERR_NOMEM;
  zn_status st = make_plan(ts, dtype, n_elems, n_tensors, chunk_bytes);
  ts->K = n_groups;
  ts->pairs = (flags & ZN_SETUP_PAIRS) ? 1 : 0;
  ts->len.assign(256ull * n_groups, 0);  // group tables are serialised with the plan
  if (ts->pairs) {                       // and so are the pair codes
    ts->packed.assign(n_groups, 0);
    ts->nF.assign(n_groups, 0);
    ts->F.assign(16ull * n_groups, 0);
    ts->tlen.assign(512ull * n_groups, 0);
  }
  if (st == ZN_OK && n_groups > 0) {
    if (!d_tensors) st = ZN_ERR_ARG;
    for (int t = 0; st == ZN_OK && t < n_tensors; t++)
      if (n_elems[t] && !d_tensors[t]) st = ZN_ERR_ARG;
    if (st == ZN_OK) st = finish_plan(ts);  // device layout is needed by the kernels
    if (st == ZN_OK) st = run_grouping(ts, d_tensors, stream);
  }
  if (st == ZN_OK) st = finish_plan(ts);
  if (st == ZN_OK) st = upload_groups(ts, stream);
  if (st != ZN_OK) {
    zn_tableset_free(ts);
    return st;
  }
  *out = ts;
  return ZN_OK;
}

zn_status zn_setup_transfer(const zn_tableset *src, const void *const *d_tensors,
                            const uint64_t *n_elems, int n_tensors, hipStream_t stream,
                            zn_tableset **out) {
  if (!out) return ZN_ERR_ARG;
  *out = nullptr;
  if (!src || src->K < 1 || !d_tensors || !n_elems || n_tensors < 1 || !on_device(src)) return ZN_ERR_ARG;
  zn_tableset *ts = new (std::nothrow) zn_tableset;
  if (!ts) return ZN_ERR_NOMEM;
  zn_status st = make_plan(ts, src->dtype, n_elems, n_tensors, src->chunk_bytes);
  if (st == ZN_OK) {
    ts->K = src->K;
    ts->len = src->len;    // the source's codes, unchanged
    ts->cost = src->cost;  // and the history of their fit
    ts->pairs = src->pairs;  // with their pair codes
    ts->packed = src->packed;
    ts->nF = src->nF;
    ts->F = src->F;
    ts->tlen = src->tlen;
    for (int t = 0; t < n_tensors; t++)
      if (n_elems[t] && !d_tensors[t]) st = ZN_ERR_ARG;
  }
  if (st == ZN_OK) st = finish_plan(ts);  // device layout for the kernels
  if (st == ZN_OK) st = run_transfer(ts, d_tensors, stream);
  if (st == ZN_OK) st = finish_plan(ts);  // hash of the new map
  if (st == ZN_OK) st = upload_groups(ts, stream);
  if (st != ZN_OK) {
    zn_tableset_free(ts);
    return st;
  }
  *out = ts;
  return ZN_OK;
}

zn_status zn_header_info(const void *h_hdr, uint64_t hdr_bytes, zn_dtype *dtype, int *n_tensors,
                         uint64_t *n_elems, uint32_t *chunk_bytes, uint32_t *n_chunks,
                         uint64_t *total_bytes, uint64_t *ts_hash) {
  const uint8_t *h = static_cast<const uint8_t *>(h_hdr);
  if (!h || hdr_bytes < 64) return ZN_ERR_ARG;
  if (get_u32(h) != kMagic || get_u16(h + 4) != kVersion || !valid_dtype(h[6]) || h[7] > 1 ||
      h[30] != kMaxLen || h[31] != ncoded(h[6]) || get_u16(h + 28) != uint32_t(segsyms(h[6])) ||
      !valid_chunk(get_u32(h + 12)) || get_u32(h + 8) < 1 || (h[7] == 0 && get_u64(h + 32) != 0))
    return ZN_ERR_CORRUPT;
  if (dtype) *dtype = zn_dtype(h[6]);
  if (n_tensors) *n_tensors = int(get_u32(h + 8));
  if (n_elems) *n_elems = get_u64(h + 16);
  if (chunk_bytes) *chunk_bytes = get_u32(h + 12);
  if (n_chunks) *n_chunks = get_u32(h + 24);
  if (total_bytes) *total_bytes = get_u64(h + 56);
  if (ts_hash) *ts_hash = get_u64(h + 32);
  return ZN_OK;
}

zn_status zn_plan_from_container(const void *d_in, uint64_t in_bytes, hipStream_t stream,
                                 zn_tableset **out) {
  if (!d_in || !out || in_bytes < 64) return ZN_ERR_ARG;
  *out = nullptr;
  uint8_t h[64];
  HIPCHK(hipMemcpyAsync(h, d_in, 64, hipMemcpyDeviceToHost, stream));
  HIPCHK(hipStreamSynchronize(stream));
  if (zn_header_info(h, 64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != ZN_OK)
    return ZN_ERR_CORRUPT;
  if (h[7] & 1) return ZN_ERR_TABLESET;
  const uint32_t T = get_u32(h + 8);
  if (64 + 16ull * T > in_bytes) return ZN_ERR_CORRUPT;
  std::vector<uint8_t> tt(16ull * T);
  HIPCHK(hipMemcpyAsync(tt.data(), static_cast<const uint8_t *>(d_in) + 64, tt.size(),
                        hipMemcpyDeviceToHost, stream));
  HIPCHK(hipStreamSynchronize(stream));
  std::vector<uint64_t> n(T);
  for (uint32_t t = 0; t < T; t++) n[t] = get_u64(tt.data() + 16 * t);
  zn_tableset *ts = new (std::nothrow) zn_tableset;
  if (!ts) return ZN_ERR_NOMEM;
  zn_status st = make_plan(ts, h[6], n.data(), int(T), get_u32(h + 12));
  if (st == ZN_ERR_ARG) st = ZN_ERR_CORRUPT;
  // the header's layout fields must be the ones this plan gives
  uint64_t ntot = 0;
  for (uint32_t t = 0; t < T; t++) ntot += n[t];
  if (st == ZN_OK && (get_u64(h + 16) != ntot || get_u32(h + 24) != ts->n_chunks || get_u64(h + 40) != ts->off_dir ||
                      get_u64(h + 48) != ts->off_records))
    st = ZN_ERR_CORRUPT;
  for (uint32_t t = 0; st == ZN_OK && t < T; t++)
    if (get_u64(tt.data() + 16 * t + 8) != ts->raw[t]) st = ZN_ERR_CORRUPT;
  if (st == ZN_OK) st = finish_plan(ts);
  if (st != ZN_OK) {
    zn_tableset_free(ts);
    return st;
  }
  *out = ts;
  return ZN_OK;
}

zn_status zn_tableset_info(const zn_tableset *ts, zn_dtype *dtype, int *n_tensors, uint64_t *h_n,
                           uint32_t *chunk_bytes, uint32_t *n_chunks, int *n_groups, uint64_t *hash) {
  if (!ts) return ZN_ERR_ARG;
  if (dtype) *dtype = zn_dtype(ts->dtype);
  if (n_tensors) *n_tensors = ts->T;
  if (h_n) memcpy(h_n, ts->n.data(), 8ull * ts->T);
  if (chunk_bytes) *chunk_bytes = ts->chunk_bytes;
  if (n_chunks) *n_chunks = ts->n_chunks;
  if (n_groups) *n_groups = ts->K;
  if (hash) *hash = ts->hash;
  return ZN_OK;
}

zn_status zn_compress_bound(const zn_tableset *ts, uint64_t *bytes) {
  if (!ts || !bytes) return ZN_ERR_ARG;
  uint64_t b = ts->off_records + 16;
  for (int t = 0; t < ts->T; t++)
    for (uint64_t i0 = 0; i0 < ts->n[t]; i0 += ts->chunk_elems) {
      const uint64_t m = std::min<uint64_t>(ts->chunk_elems, ts->n[t] - i0);
      for (int p = 0; p < ncoded(ts->dtype); p++) b += section_bytes(RAW, kbits(ts->dtype, p), m, 0, 0);
    }
  *bytes = b;
  return ZN_OK;
}

namespace {
uint64_t sizes_offset() { return kCtlBytes; }
uint64_t plans_offset(const zn_tableset *ts) { return kCtlBytes + (8ull * ts->n_chunks + 255) / 256 * 256; }
}  // namespace

zn_status zn_scratch_bytes(const zn_tableset *ts, uint64_t *bytes) {
  if (!ts || !bytes) return ZN_ERR_ARG;
  *bytes = plans_offset(ts) + uint64_t(ts->n_chunks) * plan_bytes(ts->dtype, ts->chunk_elems);
  return ZN_OK;
}

zn_status zn_compress(const zn_tableset *ts, const void *const *d_in_ptrs, void *d_out,
                      uint64_t out_cap, uint64_t *out_bytes, void *d_scratch,
                      uint64_t scratch_bytes, hipStream_t stream) {
  return zn_compress2(ts, ZN_CODER_HUFFMAN, d_in_ptrs, d_out, out_cap, out_bytes, d_scratch, scratch_bytes,
                      stream);
}

zn_status zn_compress2(const zn_tableset *ts, int coder, const void *const *d_in_ptrs, void *d_out,
                       uint64_t out_cap, uint64_t *out_bytes, void *d_scratch,
                       uint64_t scratch_bytes, hipStream_t stream) {
  if (!ts || (!d_in_ptrs && ts->n_chunks) || !d_out || !d_scratch || !on_device(ts)) return ZN_ERR_ARG;
  if (coder != ZN_CODER_HUFFMAN && (coder != ZN_CODER_TANS || ts->K > 0)) return ZN_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_scratch) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 15))
    return ZN_ERR_ARG;
  uint64_t need = 0;
  zn_scratch_bytes(ts, &need);
  if (scratch_bytes < need) return ZN_ERR_CAPACITY;
  if (out_cap < ts->off_records + 16) return ZN_ERR_CAPACITY;
  uint8_t *scr = static_cast<uint8_t *>(d_scratch);
  uint32_t *ctl = reinterpret_cast<uint32_t *>(scr);
  EncArgs a;
  a.L = dev_layout(ts);
  a.in_ptrs = reinterpret_cast<const uint8_t *const *>(d_in_ptrs);
  a.group_map = ts->K ? ts->d_map : nullptr;
  a.group_enc = ts->d_enc;
  a.group_len = ts->d_len;
  a.group_packed = ts->K ? ts->d_packed : nullptr;
  a.group_rank = ts->d_rank;
  a.group_penc = ts->d_penc;
  a.out = static_cast<uint8_t *>(d_out);
  a.plans = scr + plans_offset(ts);
  a.plan_stride = plan_bytes(ts->dtype, ts->chunk_elems);
  a.sizes = reinterpret_cast<unsigned long long *>(scr + sizes_offset());
  a.coder = coder;
  HIPCHK(launch_analyze(ts->dtype, a, stream, g_ev_before[KAnalyze], g_ev_after[KAnalyze]));
  FinishArgs f;
  f.L = a.L;
  f.dtype = ts->dtype;
  f.hdr = ts->d_hdr;
  f.hdr_bytes = uint32_t(ts->hdr.size());
  f.out = a.out;
  f.cap = out_cap;
  f.sizes = a.sizes;
  f.ctl = ctl;
  HIPCHK(launch_finish(f, stream, g_ev_before[KFinish], g_ev_after[KFinish]));
  PackArgs pk;
  pk.L = a.L;
  pk.in_ptrs = a.in_ptrs;
  pk.group_packed = a.group_packed;
  pk.group_rank = a.group_rank;
  pk.group_penc = a.group_penc;
  pk.pairs = 0;
  for (int g = 0; ts->pairs && g < ts->K; g++) pk.pairs |= ts->packed[g];
  pk.plans = a.plans;
  pk.plan_stride = a.plan_stride;
  pk.out = a.out;
  pk.ctl = ctl;
  pk.coder = coder;
  HIPCHK(launch_pack(ts->dtype, pk, stream, g_ev_before[KPack], g_ev_after[KPack]));
  if (!out_bytes) return ZN_OK;
  uint32_t flag = 0;
  uint64_t total = 0;
  HIPCHK(hipMemcpyAsync(&flag, ctl, 4, hipMemcpyDeviceToHost, stream));
  HIPCHK(hipMemcpyAsync(&total, a.out + 56, 8, hipMemcpyDeviceToHost, stream));
  HIPCHK(hipStreamSynchronize(stream));
  if (flag) return ZN_ERR_CAPACITY;
  *out_bytes = total;
  return ZN_OK;
}

}  // extern "C"

// Control area of zn_decompress_noalloc: device memory the library owns, one
// copy per GPU (each GPU holds its own copy at its own address), kept until
// the process ends.  Its need does not grow with the container: 256 bytes.
constexpr uint64_t kNoAllocScratchBytes = 256;
static_assert(kNoAllocScratchBytes >= kCtlBytes, "the decoder's control area fits");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
// The decompression launches on a caller's stream with the control area ctl
// (256 bytes: error word, group flag, sink of lanes without a whole vector).
zn_status decompress_with(const zn_tableset *ts, const void *d_in, uint64_t in_bytes,
                          void *const *d_out_ptrs, uint32_t *ctl, int sync, hipStream_t stream) {
  if (in_bytes < ts->off_records + 16) return ZN_ERR_CORRUPT;
  CheckArgs ck;
  ck.in = static_cast<const uint8_t *>(d_in);
  ck.in_bytes = in_bytes;
  ck.hdr = ts->d_hdr;
  ck.hdr_bytes = uint32_t(ts->hdr.size());
  ck.hash = ts->hash;
  ck.K = ts->K;
  ck.n_chunks = ts->n_chunks;
  ck.off_dir = ts->off_dir;
  ck.ctl = ctl;
  HIPCHK(launch_check(ck, stream, g_ev_before[KCheck], g_ev_after[KCheck]));
  DecArgs a;
  a.L = dev_layout(ts);
  a.in = ck.in;
  a.in_bytes = in_bytes;
  a.out_ptrs = reinterpret_cast<uint8_t *const *>(d_out_ptrs);
  a.group_lut = ts->d_lut;
  a.group_len = ts->d_len;
  a.group_packed = ts->K ? ts->d_packed : nullptr;
  a.K = ts->K;
  a.ctl = ctl;
  HIPCHK(launch_decode(ts->dtype, a, stream, g_ev_before[KDecode], g_ev_after[KDecode]));
  if (!sync) return ZN_OK;
  uint32_t flag = 0;
  HIPCHK(hipMemcpyAsync(&flag, ctl, 4, hipMemcpyDeviceToHost, stream));
  HIPCHK(hipStreamSynchronize(stream));
  if (flag & kErrTableset) return ZN_ERR_TABLESET;
  if (flag) return ZN_ERR_CORRUPT;
  return ZN_OK;
}

// Device address of `scratch` on each GPU, looked up once per device with
// that device current (in host code the array's name is only a stand-in).
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

zn_status noalloc_scratch(void **out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return ZN_ERR_ARG;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ZN_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZN_OK;
}
}  // namespace

extern "C" {

zn_status zn_decompress(const zn_tableset *ts, const void *d_in, uint64_t in_bytes,
                        void *const *d_out_ptrs, void *d_scratch, uint64_t scratch_bytes, int sync,
                        hipStream_t stream) {
  if (!ts || !d_in || (!d_out_ptrs && ts->n_chunks) || !d_scratch || !on_device(ts)) return ZN_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_scratch) & 15) || (reinterpret_cast<uintptr_t>(d_in) & 15))
    return ZN_ERR_ARG;
  if (scratch_bytes < kCtlBytes) return ZN_ERR_CAPACITY;
  return decompress_with(ts, d_in, in_bytes, d_out_ptrs, static_cast<uint32_t *>(d_scratch), sync, stream);
}

zn_status zn_decompress_noalloc(const zn_tableset *ts, const void *d_in, uint64_t in_bytes,
                                void *const *d_out_ptrs, uint32_t *d_status, int sync,
                                hipStream_t stream) {
  if (!ts || !d_in || (!d_out_ptrs && ts->n_chunks) || !on_device(ts)) return ZN_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_in) & 15) return ZN_ERR_ARG;
  void *ctl = nullptr;
  zn_status st = noalloc_scratch(&ctl);
  if (st != ZN_OK) return st;
  st = decompress_with(ts, d_in, in_bytes, d_out_ptrs, static_cast<uint32_t *>(ctl), sync, stream);
  // the error word, for callers that do not synchronise (a device-to-device
  // copy, stream-ordered after the kernels)
  if (d_status && (st == ZN_OK || st == ZN_ERR_CORRUPT || st == ZN_ERR_TABLESET) &&
      in_bytes >= ts->off_records + 16)
    HIPCHK(hipMemcpyAsync(d_status, ctl, 4, hipMemcpyDeviceToDevice, stream));
  return st;
}

zn_status zn_tableset_save(const zn_tableset *ts, void *h_buf, uint64_t cap, uint64_t *len) {
  if (!ts || !len) return ZN_ERR_ARG;
  *len = serial_bytes(ts);
  if (!h_buf) return ZN_OK;
  if (cap < *len) return ZN_ERR_CAPACITY;
  serialise(ts, static_cast<uint8_t *>(h_buf));
  return ZN_OK;
}

zn_status zn_tableset_load(const void *h_buf, uint64_t len, zn_tableset **out) {
  const uint8_t *b = static_cast<const uint8_t *>(h_buf);
  if (!b || !out) return ZN_ERR_ARG;
  *out = nullptr;
  if (len < 24 || get_u32(b) != kTsMagic || get_u32(b + 20) != kMaxLen) return ZN_ERR_CORRUPT;
  // version 2: with the pair codes of packed exponent pairs (BF16 with groups)
  const int ver = int(get_u16(b + 4));
  const int dt = b[6], K = b[7], T = int(get_u32(b + 12));
  const uint32_t cb = get_u32(b + 8), M = get_u32(b + 16);
  if ((ver != kVersion && ver != 2) || !valid_dtype(dt) || !valid_chunk(cb) || T < 1 || uint64_t(T) > len / 8)
    return ZN_ERR_CORRUPT;
  const int pairs = ver == 2;
  if (pairs && (dt != BF16 || K < 1)) return ZN_ERR_CORRUPT;
  const int A = alphabet0(dt);
  if (len != 24 + 8ull * T + uint64_t(K) * (A / 2) + M + (pairs ? uint64_t(K) * kTsPairBytes : 0))
    return ZN_ERR_CORRUPT;
  std::vector<uint64_t> n(T);
  for (int t = 0; t < T; t++) n[t] = get_u64(b + 24 + 8 * t);
  zn_tableset *ts = new (std::nothrow) zn_tableset;
  if (!ts) return ZN_ERR_NOMEM;
  zn_status st = make_plan(ts, dt, n.data(), T, cb);
  if (st == ZN_OK && ts->n_chunks != M) st = ZN_ERR_CORRUPT;
  if (st == ZN_OK) {
    ts->K = K;
    ts->len.assign(256ull * K, 0);
    const uint8_t *q = b + 24 + 8ull * T;
    for (int g = 0; g < K; g++)
      for (int s = 0; s < A; s += 2, q++) {
        ts->len[g * 256 + s] = *q & 15;
        ts->len[g * 256 + s + 1] = *q >> 4;
        if ((*q & 15) > kMaxLen || (*q >> 4) > kMaxLen) st = ZN_ERR_CORRUPT;
      }
    if (M) memcpy(ts->map.data(), q, M);
    q += M;
    // a plan without groups stores its map as zero bytes; with groups each
    // byte names one of the K groups
    for (uint32_t c = 0; c < M && st == ZN_OK; c++)
      if (K ? ts->map[c] >= K : ts->map[c] != 0) st = ZN_ERR_CORRUPT;
    ts->pairs = pairs;
    if (pairs) {
      ts->packed.assign(K, 0);
      ts->nF.assign(K, 0);
      ts->F.assign(16ull * K, 0);
      ts->tlen.assign(512ull * K, 0);
    }
    for (int g = 0; pairs && g < K && st == ZN_OK; g++, q += kTsPairBytes) {
      // a flag, at most 16 distinct values of F (zero past |F|), lengths
      // within the limit, no pair token past |F|, and a packing group's
      // token code complete (Kraft equality, two tokens at least)
      const int nf = q[1];
      ts->packed[g] = q[0];
      ts->nF[g] = q[1];
      memcpy(ts->F.data() + 16 * g, q + 2, 16);
      if (q[0] > 1 || nf > 16) st = ZN_ERR_CORRUPT;
      uint8_t seen[256] = {0};
      for (int i = 0; i < 16 && st == ZN_OK; i++)
        if (i < nf ? seen[q[2 + i]]++ != 0 : q[2 + i] != 0) st = ZN_ERR_CORRUPT;
      uint64_t kraft = 0;
      int d = 0;
      for (int t = 0; t < 512 && st == ZN_OK; t++) {
        const int l = (q[18 + t / 2] >> (4 * (t & 1))) & 15;
        ts->tlen[512ull * g + t] = uint8_t(l);
        if (l > kMaxLen) st = ZN_ERR_CORRUPT;
        if (t >= 256 && (((t - 256) >> 4) >= nf || ((t - 256) & 15) >= nf) && l) st = ZN_ERR_CORRUPT;
        if (l && l <= kMaxLen) {
          kraft += 1ull << (kMaxLen - l);
          d++;
        }
      }
      if (st == ZN_OK && q[0] && (d < 2 || kraft != (1ull << kMaxLen))) st = ZN_ERR_CORRUPT;
    }
  }
  if (st == ZN_ERR_ARG) st = ZN_ERR_CORRUPT;
  if (st == ZN_OK) st = finish_plan(ts);
  if (st == ZN_OK) st = upload_groups(ts, nullptr);
  if (st != ZN_OK) {
    zn_tableset_free(ts);
    return st;
  }
  *out = ts;
  return ZN_OK;
}

zn_status zn_tableset_lengths(const zn_tableset *ts, int g, uint8_t *h_len) {
  if (!ts || !h_len || g < 0 || g >= ts->K) return ZN_ERR_ARG;
  memcpy(h_len, ts->len.data() + 256ull * g, size_t(alphabet0(ts->dtype)));
  return ZN_OK;
}

zn_status zn_tableset_pairs(const zn_tableset *ts, int g, int *has_pairs, int *packed, int *n_values,
                            uint8_t *h_values, uint8_t *h_token_len) {
  if (!ts || g < 0 || g >= ts->K) return ZN_ERR_ARG;
  if (has_pairs) *has_pairs = ts->pairs;
  if (packed) *packed = ts->pairs ? ts->packed[g] : 0;
  if (n_values) *n_values = ts->pairs ? ts->nF[g] : 0;
  if (h_values) {
    memset(h_values, 0, 16);
    if (ts->pairs) memcpy(h_values, ts->F.data() + 16 * g, 16);
  }
  if (h_token_len) {
    memset(h_token_len, 0, 512);
    if (ts->pairs) memcpy(h_token_len, ts->tlen.data() + 512ull * g, 512);
  }
  return ZN_OK;
}

zn_status zn_tableset_map(const zn_tableset *ts, uint8_t *h_map) {
  if (!ts || !h_map) return ZN_ERR_ARG;
  if (ts->n_chunks) memcpy(h_map, ts->map.data(), ts->n_chunks);
  return ZN_OK;
}

zn_status zn_tableset_cost_history(const zn_tableset *ts, uint64_t *h_cost) {
  if (!ts || !h_cost) return ZN_ERR_ARG;
  for (int r = 0; r <= kRounds; r++) h_cost[r] = r < int(ts->cost.size()) ? ts->cost[r] : 0;
  return ZN_OK;
}

zn_status zn_debug_histograms(const zn_tableset *ts, const void *const *d_in_ptrs, uint32_t *d_hist,
                              hipStream_t stream) {
  if (!ts || !d_in_ptrs || !d_hist || !on_device(ts)) return ZN_ERR_ARG;
  HIPCHK(launch_hist_all(ts->dtype, dev_layout(ts), reinterpret_cast<const uint8_t *const *>(d_in_ptrs),
                         d_hist, stream));
  return ZN_OK;
}

zn_status zn_debug_code_lengths(const uint64_t *d_hist, int n, int alphabet, int group_rule,
                                uint8_t *d_len, hipStream_t stream) {
  if (!d_hist || !d_len || n < 0 || alphabet < 2 || alphabet > 256 || (alphabet & (alphabet - 1)))
    return ZN_ERR_ARG;
  HIPCHK(launch_lengths(d_hist, n, alphabet, group_rule, d_len, stream));
  return ZN_OK;
}

zn_status zn_debug_kernel_events(const char *kernel, void *before, void *after) {
  if (!kernel) return ZN_ERR_ARG;
  for (int k = 0; k < KCount; k++) {
    if (strcmp(kernel, kKernelNames[k]) == 0) {
      g_ev_before[k] = static_cast<hipEvent_t>(before);
      g_ev_after[k] = static_cast<hipEvent_t>(after);
      return ZN_OK;
    }
  }
  return ZN_ERR_ARG;
}

}  // extern "C"
