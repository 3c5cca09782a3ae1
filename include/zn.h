/*
 * zn.h -- C ABI of libzn.so, a lossless codec for floating-point tensors on
 * AMD MI355X (gfx950): exponent extraction, per-chunk order-0 histograms,
 * length-limited canonical Huffman codes, chunk-parallel decoding, and
 * NeuralZip-style grouped code tables built by a reusable setup.
 *
 * What each call computes, by source:
 *   - splitting every float into its exponent and the rest, coding the
 *     exponent and keeping sign and fraction bytes as they are: THEORY-599
 *     (nucleation note on "ZipNN: Lossless Compression for AI Models"),
 *     "What was actually shown", per-field compressibility (ZipNN Table II);
 *   - an order-0 Huffman code of the exponent per chunk: THEORY-599,
 *     order-0 only (ZipNN section III-A b);
 *   - FP8 E4M3: exponent and mantissa separated and entropy-coded
 *     independently: "Lossless Compression of Neural Network Components:
 *     Weights, Checkpoints, and K/V Caches in Low-Precision Formats",
 *     Abstract;
 *   - grouping chunks with similar exponent distributions, sharing their
 *     Huffman codes, and choosing these in a setup that later encodings reuse
 *     while still reading the current values; bit-exact reconstruction:
 *     "NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract.
 *
 * Conventions for every call:
 *   - Pointers named d_* are device memory owned by the caller (for example
 *     torch tensors).  h_* are host memory.  The library owns only the opaque
 *     zn_tableset and the device memory inside it.
 *   - zn_compress and zn_decompress allocate nothing; they launch on the
 *     caller's stream in stream order and need d_scratch of at least
 *     zn_scratch_bytes() bytes (16-byte aligned).  Concurrent calls on one
 *     tableset need distinct scratch buffers.
 *   - A tableset's device memory lives on the device that was current when
 *     the tableset was made.  Every call that launches work with it needs
 *     that device current (ZN_ERR_ARG otherwise); zn_tableset_free may be
 *     called with any device current.
 *   - Inputs are read-only; outputs must not overlap inputs.  Tensor data
 *     pointers should be 16-byte aligned (unaligned ones take a slow path).
 *   - Calls return a zn_status and never throw.  HIP failures map to
 *     ZN_ERR_HIP.  A corrupt container gives ZN_ERR_CORRUPT and leaves the
 *     outputs unspecified; it never makes the library read or write outside
 *     the buffers it was given.
 *   - Bitstreams are bit-identical to the CPU oracle's for the same inputs.
 */
#ifndef ZN_H
#define ZN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ZN_FP4X2_E2M1: every element is one byte holding two FP4 E2M1 values, the
 * first in the low nibble (a nibble is sign | 2 exponent bits | 1 mantissa
 * bit); element counts are bytes.  The byte's two exponents form one coded
 * 4-bit field and its two mantissas one coded 2-bit field; its two sign bits
 * are kept raw. */
typedef enum { ZN_BF16 = 0, ZN_FP32 = 1, ZN_FP8_E4M3 = 2, ZN_FP4X2_E2M1 = 3 } zn_dtype;

typedef enum {
  ZN_OK = 0,
  ZN_ERR_ARG = -1,       /* bad argument (null pointer, size, dtype, chunk size) */
  ZN_ERR_CORRUPT = -2,   /* container fails a structural or bitstream check      */
  ZN_ERR_CAPACITY = -3,  /* output or scratch buffer too small                    */
  ZN_ERR_TABLESET = -4,  /* container needs another tableset (hash mismatch)     */
  ZN_ERR_HIP = -5,       /* a HIP runtime call failed                             */
  ZN_ERR_NOMEM = -6      /* host or setup-time device allocation failed           */
} zn_status;

/* A plan for a fixed list of tensor sizes: dtype, chunk size, the container
 * layout, and optionally K grouped code tables.  Library-owned. */
/* Entropy coder of the exponent stream (zn_compress2).  ZN_CODER_TANS is the
 * tabled asymmetric-numeral-system coder (FSE) that THEORY-599's order-0
 * discussion reports, after ZipNN Fig. 4, as coding exponents 0-2% smaller
 * than Huffman; it serves chunks coded with their own table (plans without
 * groups).  The other coded fields keep their Huffman codes. */
typedef enum { ZN_CODER_HUFFMAN = 0, ZN_CODER_TANS = 1 } zn_coder;

typedef struct zn_tableset zn_tableset;

/* zn_setup -- the reusable setup ("NeuralZip", Abstract).
 *   n_elems[n_tensors]: element count of each tensor (host array).
 *   chunk_bytes: uncompressed bytes per chunk; a multiple of 4096 in
 *     [4096, 1 MiB].  Chunks never span tensors.
 *   n_groups == 0: per-chunk code tables only; d_tensors may be NULL and no
 *     kernel runs.  n_groups in [1, 255]: every chunk of the given tensors is
 *     histogrammed on the GPU, chunks are grouped by their exponent
 *     histograms (integer Lloyd rounds) and each group gets one shared code;
 *     d_tensors (host array of device pointers) must then be valid.
 * Allocates device memory for the plan (this is the only call that does,
 * with zn_setup_transfer, zn_plan_from_container and zn_tableset_load).
 * Synchronises stream. */
zn_status zn_setup(zn_dtype dtype, const void *const *d_tensors, const uint64_t *n_elems,
                   int n_tensors, uint32_t chunk_bytes, int n_groups, hipStream_t stream,
                   zn_tableset **out);

/* zn_setup2 -- zn_setup with flags.  ZN_SETUP_PAIRS: packed exponent pairs
 * ("NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract:
 * recurring exponent tuples represented by packed exponents, chosen by the
 * setup).  After the grouping, each group's 16 most common exponent values
 * (F) are found, the group's tokens are counted on the GPU -- in every
 * 32-value strip of a chunk's exponents, values 2i and 2i+1 both in F make
 * one pair token, every other value a single token -- each group gets an
 * optimal code (lengths <= 11) over its 512 tokens, and it packs when that
 * code takes fewer bits than its single-value code on its own chunks.
 * zn_compress then codes a packing group's chunks with tokens, and
 * zn_decompress reads them.  BF16 with n_groups >= 1 only (ZN_ERR_ARG
 * otherwise, and for unknown flags).  The saved tableset is format version 2.
 * Everything else as zn_setup. */
enum { ZN_SETUP_PAIRS = 1 };
zn_status zn_setup2(zn_dtype dtype, const void *const *d_tensors, const uint64_t *n_elems,
                    int n_tensors, uint32_t chunk_bytes, int n_groups, int flags, hipStream_t stream,
                    zn_tableset **out);

/* zn_setup_transfer -- a setup reused on other tensors of the same dtype and
 * chunk size, such as another architecture of the same kind ("NeuralZip: Reusable
 * Setup for Fast Lossless Compression", Abstract).  The new plan keeps src's
 * K group codes unchanged; every chunk of the new tensors (d_tensors: host
 * array of device pointers; n_elems[n_tensors] host) is histogrammed on the
 * GPU and assigned by its content to the group code that codes its exponent
 * stream in the fewest bits, ties to the smaller group id; a chunk that every
 * group code lacks a symbol for goes to group 0 and is coded with its own
 * table when compressed.  The cost history is src's.  src must have groups
 * (ZN_ERR_ARG otherwise) and stays valid.  Allocates device memory for the
 * plan; synchronises stream. */
zn_status zn_setup_transfer(const zn_tableset *src, const void *const *d_tensors,
                            const uint64_t *n_elems, int n_tensors, hipStream_t stream,
                            zn_tableset **out);

/* zn_header_info -- the facts a container's 64-byte header records, read
 * from host memory (h_hdr, hdr_bytes >= 64; nothing past byte 64 is read):
 * dtype, tensor count, total element count, chunk size, chunk count, total
 * container bytes and the tableset hash (0 unless the container was made with
 * group tables).  Host-only: no HIP call, usable without a GPU.  A decoder
 * learns from it which plan and tableset it needs before any device work
 * ("NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract: the
 * representations chosen by the setup are what later encodings use, so a
 * container must name the setup it depends on).  ZN_ERR_ARG for a null or
 * short buffer; ZN_ERR_CORRUPT when the magic, version, dtype, flags, chunk
 * size, segment size, code-length limit, coded-stream count or tensor count
 * is not one this library writes, or the hash is set without the group flag.
 * Any output pointer may be NULL. */
zn_status zn_header_info(const void *h_hdr, uint64_t hdr_bytes, zn_dtype *dtype, int *n_tensors,
                         uint64_t *n_elems, uint32_t *chunk_bytes, uint32_t *n_chunks,
                         uint64_t *total_bytes, uint64_t *ts_hash);

/* zn_plan_from_container -- a plan (without groups) that matches the layout
 * of an existing container; reads its header and tensor table with two
 * synchronous copies and checks that the header's layout fields (element
 * total, chunk count, directory, record and raw-plane offsets) are the ones
 * that plan gives (ZN_ERR_CORRUPT otherwise).  Containers that use group
 * tables need the tableset they were compressed with (ZN_ERR_TABLESET here).
 * ZN_ERR_ARG for null pointers or in_bytes < 64. */
zn_status zn_plan_from_container(const void *d_in, uint64_t in_bytes, hipStream_t stream,
                                 zn_tableset **out);

/* Plan facts.  Any output pointer may be NULL; h_n_elems gets n_tensors values. */
zn_status zn_tableset_info(const zn_tableset *ts, zn_dtype *dtype, int *n_tensors,
                           uint64_t *h_n_elems, uint32_t *chunk_bytes, uint32_t *n_chunks,
                           int *n_groups, uint64_t *hash);

/* Worst-case container size for the plan's tensors (host-only arithmetic). */
zn_status zn_compress_bound(const zn_tableset *ts, uint64_t *bytes);

/* Device scratch needed by zn_compress / zn_decompress for this plan: 256
 * control bytes, 8 bytes per chunk (record sizes) and a code plan per chunk
 * of 64 + 1024 bytes per coded field (the code chosen for each stream) plus
 * 2 bytes per segment of the exponent stream (tANS segment lengths): at
 * 256 KiB chunks 1/163 of the input for BF16, 1/56 for FP32.
 * Decompression alone needs only the first 256 bytes. */
zn_status zn_scratch_bytes(const zn_tableset *ts, uint64_t *bytes);

/* zn_compress -- one container holding every tensor of the plan.  Per chunk
 * and coded field: the order-0 histogram, an optimal prefix code of the field
 * (THEORY-599, nucleation note on ZipNN, "What was actually shown": the
 * exponent is extracted and Huffman-coded order-0 while sign and fraction
 * bytes stay as they are, ZipNN Table II and section III-A b), or the group's
 * shared code chosen by the setup ("NeuralZip: Reusable Setup for Fast
 * Lossless Compression", Abstract), then the packed bits.
 *   d_in_ptrs: DEVICE array of n_tensors device pointers to the tensors.
 *   d_out / out_cap: output buffer; out_cap >= zn_compress_bound() always fits.
 *   out_bytes: host; if non-NULL the call synchronises the stream and returns
 *     the container size (and ZN_ERR_CAPACITY if it did not fit).  If NULL
 *     the call is asynchronous; the size is the u64 at d_out + 56 and the
 *     capacity flag is the u32 at d_scratch once the stream has finished.
 * Per-chunk tables when the plan has no groups; with groups, chunk c uses
 * its group's shared code unless the chunk holds a symbol that code lacks
 * (an escape), which is then coded with its own table. */
zn_status zn_compress(const zn_tableset *ts, const void *const *d_in_ptrs, void *d_out,
                      uint64_t out_cap, uint64_t *out_bytes, void *d_scratch,
                      uint64_t scratch_bytes, hipStream_t stream);

/* zn_compress2 -- zn_compress with the exponent stream's coder chosen
 * (zn_coder; zn_compress is ZN_CODER_HUFFMAN).  With ZN_CODER_TANS each
 * chunk's exponent stream gets normalised counts summing to 2^11 and is
 * coded with tabled ANS (THEORY-599, order-0 discussion; ZipNN Fig. 4), when
 * that section is smaller than the raw one; a constant stream stays constant.
 * Every segment is encoded twice (once to size it, once to write it) and
 * decoding takes one table step per symbol, so tANS trades speed for the
 * pages' 0-2%.  Arguments, ownership, synchronisation and errors as
 * zn_compress; ZN_ERR_ARG for an unknown coder or for ZN_CODER_TANS with a
 * plan that has groups (group codes are Huffman codes).  zn_decompress reads
 * either coder's containers. */
zn_status zn_compress2(const zn_tableset *ts, int coder, const void *const *d_in_ptrs, void *d_out,
                       uint64_t out_cap, uint64_t *out_bytes, void *d_scratch,
                       uint64_t scratch_bytes, hipStream_t stream);

/* zn_decompress -- exact reconstruction of every tensor of the container
 * (bit-to-bit: "NeuralZip: Reusable Setup for Fast Lossless Compression",
 * Abstract; lossless: "Lossless Compression of Neural Network Components ...
 * in Low-Precision Formats", Abstract): chunks and their segments decode in
 * parallel and the coded fields are merged back with the stored bits.
 *   d_out_ptrs: DEVICE array of n_tensors device pointers, each large enough
 *     for its tensor.
 *   sync != 0: synchronises and returns ZN_ERR_CORRUPT if any check failed.
 *   sync == 0: asynchronous; the u32 at d_scratch is non-zero afterwards if
 *     a check failed.
 * The plan must match the container's layout; a container built with group
 * tables needs the same tableset (checked through its hash). */
zn_status zn_decompress(const zn_tableset *ts, const void *d_in, uint64_t in_bytes,
                        void *const *d_out_ptrs, void *d_scratch, uint64_t scratch_bytes,
                        int sync, hipStream_t stream);

/* zn_decompress_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): zn_decompress with the same kernels and checks, its 256-byte
 * control area (error word, group flag, sink of lanes without a whole
 * vector) in a static device array owned by the library instead of caller
 * scratch.  Allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Each GPU holds its own copy of the array until the process ends;
 * every call on a GPU shares that GPU's copy, which keeps the last call's
 * contents (the first kernel of each call overwrites what it needs), so
 * calls that overlap on one GPU (several streams or host threads) race and
 * must be ordered by the caller.  The area's size does not depend on the
 * container, so no container is refused for its size.
 *   d_status: NULL, or a caller-owned device u32 that receives the error word
 *     (0 ok, 2 corrupt, 4 tableset mismatch) by a device-to-device copy
 *     ordered after the kernels, for callers that do not synchronise.
 *   sync: as for zn_decompress.  Other arguments and statuses as for
 *     zn_decompress. */
zn_status zn_decompress_noalloc(const zn_tableset *ts, const void *d_in, uint64_t in_bytes,
                                void *const *d_out_ptrs, uint32_t *d_status, int sync,
                                hipStream_t stream);

/* Serialisation of a plan, byte-identical to the CPU oracle's; its FNV-1a-64
 * hash is what containers record. */
zn_status zn_tableset_save(const zn_tableset *ts, void *h_buf, uint64_t cap, uint64_t *len);
zn_status zn_tableset_load(const void *h_buf, uint64_t len, zn_tableset **out);
/* Group g's code lengths (alphabet of the exponent stream) and the chunk map. */
zn_status zn_tableset_lengths(const zn_tableset *ts, int g, uint8_t *h_len);
/* Group g's packed-pair code (host outputs, any may be NULL): has_pairs = 1
 * if the setup was made with ZN_SETUP_PAIRS; packed = 1 if the group packs;
 * n_values = |F|; h_values[16] = F by rank (zero past |F|); h_token_len[512]
 * = token code lengths (singles 0..255, pair 256 + 16*rank(x) + rank(y)). */
zn_status zn_tableset_pairs(const zn_tableset *ts, int g, int *has_pairs, int *packed, int *n_values,
                            uint8_t *h_values, uint8_t *h_token_len);
zn_status zn_tableset_map(const zn_tableset *ts, uint8_t *h_map);
/* Setup objective (total coded exponent bits) before each of the 8 Lloyd
 * rounds and after the last one: h_cost[9]. */
zn_status zn_tableset_cost_history(const zn_tableset *ts, uint64_t *h_cost);
void zn_tableset_free(zn_tableset *ts);

const char *zn_status_str(zn_status s);

/* ---- single steps, for parity tests of each stage (asynchronous) ----
 * zn_debug_histograms: order-0 histograms of every coded stream of every
 *   chunk of the plan: d_hist[n_chunks][n_coded][256] u32.
 * zn_debug_code_lengths: code lengths of n histograms (d_hist[n][256] u64)
 *   by the device package-merge; group_rule != 0 applies the group-table
 *   rule for single-symbol histograms; d_len[n][256]. */
zn_status zn_debug_histograms(const zn_tableset *ts, const void *const *d_in_ptrs,
                              uint32_t *d_hist, hipStream_t stream);
zn_status zn_debug_code_lengths(const uint64_t *d_hist, int n, int alphabet, int group_rule,
                                uint8_t *d_len, hipStream_t stream);

/* ---- kernel timing, for measurement tools ----
 * zn_debug_kernel_events: from now on, every launch of the named kernel
 *   ("analyze", "finish", "pack" (compression), "check", "decode"
 *   (decompression)) sets the HIP events `before` and `after` (hipEvent_t,
 *   created with timing by the caller, who owns them) to its start and end
 *   times.  The events ride on the kernel's own dispatch, so no marker is
 *   added to the stream between launches; a call that launches nothing (no
 *   chunks) leaves them as they were.  NULL events stop the timing of that
 *   kernel.  Process-wide, not thread-safe; ZN_ERR_ARG for an unknown name. */
zn_status zn_debug_kernel_events(const char *kernel, void *before, void *after);

#ifdef __cplusplus
}
#endif
#endif
