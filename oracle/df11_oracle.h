/*
 * Reference ("oracle") implementation of DFloat11-style lossless BF16 weight
 * compression: a plain, slow, single-threaded C encoder and a bit-serial
 * decoder.  TEST INFRASTRUCTURE ONLY.  The product library never includes,
 * links or calls this code; only the test suite, the smoke check and the
 * benchmark's CPU-baseline timing do.
 *
 * What the method computes (mlx-dfloat project page, introduction and its
 * 16-bit weight diagram): each BF16 word is split into its 8-bit exponent,
 * which is replaced by a variable-length prefix code, and its sign + 7-bit
 * fraction, which is kept as one raw byte.  Decoding must give back every
 * word bit for bit (same page, introduction and "Status", milestone 1).
 *
 * The container layout written here is this project's own (version 4); its
 * fields are documented next to the writer in df11_oracle.c.
 */
#ifndef DF11_ORACLE_H
#define DF11_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_E_ARG = 1,       /* bad argument (NULL, capacity too small, ...) */
    ORACLE_E_FORMAT = 2,    /* container structure is invalid */
    ORACLE_E_CORRUPT = 3,   /* bitstream holds no valid code at some point */
    ORACLE_E_TRUNCATED = 4  /* bitstream ends before all codes are read */
};

/* Optimal prefix-code lengths under a maximum length `cap` by package-merge.
 * freq[256] in, len[256] out (0 = symbol absent).  Returns ORACLE_OK. */
int oracle_code_lengths(const uint64_t *freq, int cap, uint8_t *len);

/* Canonical code values for a length vector (codes sorted by (length, symbol),
 * first code 0).  code[256] out; entries of absent symbols are 0. */
int oracle_canonical_codes(const uint8_t *len, uint32_t *code);

/* Upper bound on the container size for n words. */
uint64_t oracle_container_bound(uint64_t n);

/* Header flag: the header holds the SHA-256 of the source words. */
#define ORACLE_FLAG_SHA256 1u

/* Encode n BF16 words (as uint16) into a version-4 container.
 * dims[ndim] is the tensor shape (ndim <= 8, product must equal n).
 * Returns ORACLE_OK and the container size in *out_bytes. */
int oracle_encode(const uint16_t *words, uint64_t n, int ndim, const uint64_t *dims,
                  uint8_t *out, uint64_t out_cap, uint64_t *out_bytes);

/* The same with header flags (0 or ORACLE_FLAG_SHA256). */
int oracle_encode_flags(const uint16_t *words, uint64_t n, int ndim, const uint64_t *dims, uint32_t flags,
                        uint8_t *out, uint64_t out_cap, uint64_t *out_bytes);

/* SHA-256 (FIPS 180-4) of len bytes; the 32-byte digest to out. */
void oracle_sha256(const uint8_t *msg, uint64_t len, uint8_t out[32]);

/* Bit-serial decode of a whole container: reads one bit at a time through
 * the canonical table, ignores the chunk and window index.  out[n]. */
int oracle_decode(const uint8_t *c, uint64_t bytes, uint16_t *out, uint64_t n);

/* Decode one chunk, starting from its start_bit alone (chunk index only). */
int oracle_decode_chunk(const uint8_t *c, uint64_t bytes, uint64_t chunk, uint16_t *out);

/* Decode the codes of one window of a chunk from its (gap, cnt) entries.
 * Writes the cnt decoded words to out, cnt to *n_out and the end bit
 * position to *end_bit. */
int oracle_decode_window(const uint8_t *c, uint64_t bytes, uint64_t chunk, int win,
                       uint16_t *out, uint64_t *n_out, uint64_t *end_bit);

/* Structural check of a container (header fields, Kraft sum, chunk index
 * against a re-walk of the stream, window index against the code starts);
 * with the SHA-256 flag, also the stored hash against the hash of the
 * decoded words (ORACLE_E_CORRUPT when they differ). */
int oracle_check(const uint8_t *c, uint64_t bytes);

#ifdef __cplusplus
}
#endif
#endif
