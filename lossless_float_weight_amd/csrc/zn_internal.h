// zn_internal.h -- launch interface between the C ABI (zn_api.hip) and the
// kernels (zn_encode.hip, zn_decode.hip, zn_setup.hip).  Not installed.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zn_common.h"

namespace zn {

struct EncArgs {
  DevLayout L;
  const uint8_t *const *in_ptrs;   // [T] device pointers
  const uint8_t *group_map;        // [n_chunks] or nullptr
  const uint32_t *group_enc;       // [K][256] bit-reversed code | len << 16
  const uint8_t *group_len;        // [K][256]
  const uint8_t *group_packed;     // [K] 1: the group codes packed exponent pairs (BF16)
  const uint8_t *group_rank;       // [K][256] rank of a value in the group's F, or 0xFF
  const uint32_t *group_penc;      // [K][256] pair token codes, as group_enc
  uint8_t *out;                    // container (the raw planes are written here)
  uint8_t *plans;                  // [n_chunks][plan_stride] code choice and code words
  uint64_t plan_stride;            // plan_bytes(dtype, chunk_elems)
  unsigned long long *sizes;       // [n_chunks] record bytes
  int coder;                       // Coder of the exponent stream (TANS: no group tables)
};
// Packs every record at its directory offset (after k_finish).
struct PackArgs {
  DevLayout L;
  const uint8_t *const *in_ptrs;
  const uint8_t *group_packed;     // as in EncArgs
  const uint8_t *group_rank;
  const uint32_t *group_penc;
  int pairs;                       // some group packs exponent pairs
  const uint8_t *plans;
  uint64_t plan_stride;
  uint8_t *out;
  const uint32_t *ctl;             // [0] non-zero: the container did not fit, write nothing
  int coder;
};

// Offsets of the records (exclusive scan of their sizes), the directory, the
// header and the alignment gaps; one workgroup.
struct FinishArgs {
  DevLayout L;
  int dtype;
  const uint8_t *hdr;              // header template (64 + 16T bytes, total = 0)
  uint32_t hdr_bytes;
  uint8_t *out;
  uint64_t cap;
  const unsigned long long *sizes;
  uint32_t *ctl;                   // [0] error bits
};

struct DecArgs {
  DevLayout L;
  const uint8_t *in;
  uint64_t in_bytes;
  uint8_t *const *out_ptrs;        // [T] device pointers
  const uint32_t *group_lut;       // [K][2048]
  const uint8_t *group_len;        // [K][256]
  const uint8_t *group_packed;     // [K] 1: one token per table entry (packed pairs)
  int K;
  uint32_t *ctl;                   // [0] error bits
};

struct CheckArgs {
  const uint8_t *in;
  uint64_t in_bytes;
  const uint8_t *hdr;              // expected header + tensor table
  uint32_t hdr_bytes;
  uint64_t hash;                   // tableset hash (groups) or 0
  int K;
  uint32_t n_chunks;
  uint64_t off_dir;
  uint32_t *ctl;
};

// Error bits in ctl[0].
constexpr uint32_t kErrCapacity = 1, kErrCorrupt = 2, kErrTableset = 4;
// Compress scratch: ctl[0..63] control, record sizes, then one plan per chunk.
constexpr uint64_t kCtlBytes = 256;
// Bytes [128, 144) of the decompress scratch take the stores of lanes that
// have nothing to store (their content is meaningless).
constexpr uint64_t kSinkOff = 128;

// bytes of one chunk's plan (compress scratch) for chunks of chunk_elems elements
uint64_t plan_bytes(int dtype, uint32_t chunk_elems);
// e0, e1 (optional): events that take the start and end times of the
// launch, attached to its dispatch (no marker joins the stream); left as they
// were when there is nothing to launch.
hipError_t launch_analyze(int dtype, const EncArgs &a, hipStream_t s, hipEvent_t e0 = nullptr,
                          hipEvent_t e1 = nullptr);
hipError_t launch_finish(const FinishArgs &a, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_pack(int dtype, const PackArgs &a, hipStream_t s, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr);
hipError_t launch_check(const CheckArgs &a, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_decode(int dtype, const DecArgs &a, hipStream_t s, hipEvent_t e0 = nullptr,
                         hipEvent_t e1 = nullptr);

// setup
hipError_t launch_hist_all(int dtype, const DevLayout &L, const uint8_t *const *in_ptrs,
                           uint32_t *hist /* [n_chunks][ncoded][256] */, hipStream_t s);
hipError_t launch_hist0(int dtype, const DevLayout &L, const uint8_t *const *in_ptrs,
                        uint32_t *hist /* [n_chunks][256], the first coded stream */, hipStream_t s);
hipError_t launch_pool(const uint32_t *hist, int stride_words, int A, uint32_t M, const uint8_t *map,
                       unsigned long long *pooled /* [K][256] */, int K, hipStream_t s);
hipError_t launch_lengths(const uint64_t *hw, int n, int A, int group_rule, uint8_t *len,
                          hipStream_t s);
hipError_t launch_group_tables(const uint8_t *len, int K, int A, uint32_t *enc, uint32_t *lut,
                               uint32_t *ctl, hipStream_t s);
hipError_t launch_assign(const uint32_t *hist, int stride_words, int A, uint32_t M, const uint8_t *len,
                         int K, int reassign, uint8_t *map, unsigned long long *cost, hipStream_t s);
hipError_t launch_keys(const uint32_t *hist, int stride_words, int A, const DevLayout &L,
                       unsigned long long *keys, hipStream_t s);
// packed exponent pairs (BF16): F, ranks, token counts and lengths, packing flags
hipError_t launch_pairs(const DevLayout &L, const uint8_t *const *in_ptrs, const uint8_t *map,
                        const unsigned long long *pooled /* [K][256] */, const uint8_t *len /* [K][256] */,
                        int K, uint8_t *F /* [K][16] */, uint8_t *nF /* [K] */, uint8_t *rank /* [K][256] */,
                        unsigned long long *tok /* [K][512], zeroed */, uint8_t *tlen /* [K][512] */,
                        uint8_t *packed /* [K] */, hipStream_t s);
// a packing group's tables: len/enc take the single tokens, penc the pairs,
// lut the one-token decode table; non-packing groups are left alone
hipError_t launch_pair_tables(const uint8_t *tlen, const uint8_t *F, const uint8_t *packed, int K, uint8_t *len,
                              uint32_t *enc, uint32_t *penc, uint32_t *lut, uint32_t *ctl, hipStream_t s);

}  // namespace zn
