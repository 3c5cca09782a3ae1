/*
 * zno.h -- CPU oracle of the exponent-Huffman float codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load liboracle_zno.so.  The GPU library
 * (libzn.so) never links, loads or includes anything from this directory,
 * and this directory includes nothing from it: the format constants below
 * are restated here on purpose.
 *
 * What is computed, and where it comes from:
 *   - field split of each float into its biased exponent and the rest:
 *     THEORY-599 (nucleation note on ZipNN), "What was actually shown",
 *     per-field compressibility (ZipNN Table II): the exponent is extracted,
 *     the sign and fraction bytes are kept as they are;
 *     FP8: "Lossless Compression of Neural Network Components ... in
 *     Low-Precision Formats", Abstract: exponent and mantissa are separated
 *     and entropy-coded independently.
 *   - order-0 Huffman coding of the exponent per chunk: THEORY-599,
 *     "Order-0 only (ZipNN section III-A b)".
 *   - grouped chunks sharing Huffman tables, chosen by a reusable setup:
 *     "NeuralZip: Reusable Setup for Fast Lossless Compression", Abstract.
 * Everything the pages leave open (code-length limit, segment size, bit
 * order, container) is fixed by the format description in this header's
 * companion zno.c, one reading per comment.
 */
#ifndef ZNO_H
#define ZNO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ZNO_FP4X2_E2M1: one element is a byte holding two FP4 E2M1 values, the
 * first in the low nibble; element counts are bytes. */
enum { ZNO_BF16 = 0, ZNO_FP32 = 1, ZNO_FP8_E4M3 = 2, ZNO_FP4X2_E2M1 = 3 };
enum { ZNO_OK = 0, ZNO_ERR_ARG = -1, ZNO_ERR_CORRUPT = -2, ZNO_ERR_CAPACITY = -3,
       ZNO_ERR_TABLESET = -4, ZNO_ERR_NOMEM = -6 };
enum { ZNO_RAW = 0, ZNO_CONST = 1, ZNO_HUFF = 2, ZNO_GROUP = 3, ZNO_TANS = 4 };
/* Coder of the exponent stream (stream 0) of chunks coded with their own
 * table: canonical Huffman (the default) or tabled asymmetric numeral
 * systems (tANS) with 2^11 states. */
enum { ZNO_CODER_HUFFMAN = 0, ZNO_CODER_TANS = 1 };
#define ZNO_TANS_LOG 11

typedef struct zno_tableset zno_tableset;

/* Per-call diagnostics (not part of the format). */
typedef struct {
  uint64_t mode_count[4][5];   /* [coded stream][mode] */
  uint64_t stream_bytes[4];    /* record bytes per coded stream, headers included */
  uint64_t payload_bits[4];    /* Huffman/raw payload bits per coded stream */
  uint64_t raw_plane_bytes;    /* always-raw section bytes */
  uint64_t escapes;            /* chunks whose group table missed a symbol */
} zno_stats;

/* ---- single steps, exported so tests can pin each one ---- */
void zno_split(int dtype, const void *in, uint64_t n, uint8_t *planes /* [n_coded][n] */,
               uint8_t *rawbits /* [n]: BF16 sign+fraction byte, FP8 sign bit, FP32 unused */);
void zno_merge(int dtype, const uint8_t *planes, const uint8_t *rawbits, uint64_t n, void *out);
int  zno_code_lengths(const uint64_t *hist, int alphabet, int max_len, uint8_t *len);
int  zno_group_lengths(const uint64_t *hist, int alphabet, int max_len, uint8_t *len);
void zno_canonical_codes(const uint8_t *len, int alphabet, int max_len, uint32_t *code);

/* tANS steps: normalised counts (sum 2^11, at least 1 for every present
 * symbol), the spread of symbols over the 2^11 states, and one segment's
 * encoding (symbols in decoding order; returns its bit count, writes the
 * final state minus 2^11, and the bits LSB-first to out when non-NULL). */
int  zno_tans_normalize(const uint64_t *hist, int alphabet, uint32_t *q);
void zno_tans_spread(const uint32_t *q, int alphabet, uint8_t *sym_of_state);
int64_t zno_tans_encode(const uint32_t *q, int alphabet, const uint8_t *sym, uint64_t n,
                        uint8_t *out, uint32_t *final_state);
int  zno_tans_decode(const uint32_t *q, int alphabet, const uint8_t *bits, uint64_t nbits,
                     uint32_t final_state, uint64_t n, uint8_t *sym);

/* ---- container ---- */
int zno_compress_bound(int dtype, const uint64_t *n_elems, int n_tensors, uint32_t chunk_bytes,
                       uint64_t *bound);
int zno_compress(int dtype, const void *const *tensors, const uint64_t *n_elems, int n_tensors,
                 uint32_t chunk_bytes, const zno_tableset *ts, void *out, uint64_t cap,
                 uint64_t *out_bytes, zno_stats *stats);
/* zno_compress with a coder for the exponent stream (ZNO_CODER_*); tANS only
 * without group tables (ZNO_ERR_ARG otherwise). */
int zno_compress2(int dtype, const void *const *tensors, const uint64_t *n_elems, int n_tensors,
                  uint32_t chunk_bytes, const zno_tableset *ts, int coder, void *out, uint64_t cap,
                  uint64_t *out_bytes, zno_stats *stats);
int zno_header(const void *in, uint64_t in_bytes, int *dtype, int *n_tensors, uint64_t *n_total,
               uint32_t *chunk_bytes, uint32_t *n_chunks, uint64_t *total_bytes, uint64_t *ts_hash);
int zno_decompress(const void *in, uint64_t in_bytes, const zno_tableset *ts, void *const *outs,
                   const uint64_t *n_elems, int n_tensors);

/* One chunk record alone (for sampled checks of large containers). */
int zno_encode_chunk(int dtype, const void *chunk, uint64_t n, const uint8_t *group_len /* or NULL */,
                     int group_id, void *rec, uint64_t cap, uint64_t *rec_bytes, int *escape);
int zno_encode_chunk2(int dtype, const void *chunk, uint64_t n, const uint8_t *group_len, int group_id,
                      int coder, void *rec, uint64_t cap, uint64_t *rec_bytes, int *escape);

/* ---- NeuralZip-style setup ---- */
int zno_setup(int dtype, const void *const *tensors, const uint64_t *n_elems, int n_tensors,
              uint32_t chunk_bytes, int n_groups, zno_tableset **out);
/* zno_setup with flags: ZNO_SETUP_PAIRS adds the packed exponent pairs of
 * R9 (BF16 with groups only; ZNO_ERR_ARG otherwise). */
enum { ZNO_SETUP_PAIRS = 1 };
int zno_setup2(int dtype, const void *const *tensors, const uint64_t *n_elems, int n_tensors,
               uint32_t chunk_bytes, int n_groups, int flags, zno_tableset **out);
/* The source's group codes for other tensors of its dtype and chunk size;
 * each chunk to the group code of least coded size (content, not position). */
int zno_setup_transfer(const zno_tableset *src, const void *const *tensors, const uint64_t *n_elems,
                       int n_tensors, zno_tableset **out);
void zno_tableset_free(zno_tableset *ts);
int zno_tableset_info(const zno_tableset *ts, int *n_groups, uint32_t *n_chunks, uint64_t *hash);
int zno_tableset_lengths(const zno_tableset *ts, int g, uint8_t *len /* alphabet */);
int zno_tableset_map(const zno_tableset *ts, uint8_t *map /* n_chunks */);
int zno_tableset_cost_history(const zno_tableset *ts, uint64_t *cost /* rounds+1 */);
/* R9: group g's packing flag, |F|, F[16] and its 512 token lengths; returns
 * 1 if the setup has pair codes, 0 if not. */
int zno_tableset_pairs(const zno_tableset *ts, int g, int *packed, int *nF, uint8_t *F, uint8_t *tlen);
int zno_tableset_save(const zno_tableset *ts, void *buf, uint64_t cap, uint64_t *len);
int zno_tableset_load(const void *buf, uint64_t len, zno_tableset **out);

#ifdef __cplusplus
}
#endif
#endif
