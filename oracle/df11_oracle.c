/*
 * Oracle for DFloat11-style lossless BF16 compression.  TEST INFRASTRUCTURE
 * ONLY: the product library never includes, links or calls this file.
 *
 * Plain, slow, obviously-correct C.  One tensor at a time, one thread, one
 * bit at a time where bits are read.  Each function names the passage of the
 * source pages it follows.
 *
 * Sources:
 *  - mlx-dfloat project page, introduction and the 16-bit weight diagram:
 *    a BF16 weight is sign | 8 exponent bits | 7 fraction bits; the exponent
 *    is replaced by a variable-length code ("the same idea a zip file uses"),
 *    sign + fraction are kept as one raw byte.
 *  - same page, introduction and "Status" (milestone 1): decoding gives the
 *    original BF16 words bit for bit.
 *  - df11pack project page, "Beyond the official format" (--luts=correct):
 *    table entries that no valid stream can reach are defined as zero; and
 *    "Use" (verify): structure, sampled chunks, or full decode.
 *
 * Where the pages are silent (which prefix code, tie-breaks, bit order,
 * chunking, windows, padding) this file takes one fixed reading:
 *  - code: optimal prefix code with maximum length 24, by package-merge
 *    (Larmore and Hirschberg 1990); leaves sorted by (frequency, symbol);
 *    on equal weight a leaf is taken before a package;
 *  - canonical code values: symbols sorted by (length, symbol), first code 0,
 *    next = (code + 1) << (next length - this length)  (the deflate
 *    construction, RFC 1951 section 3.2.2);
 *  - bitstream: codes concatenated most significant bit first; bit 7 of byte
 *    0 is the first bit;
 *  - raw byte: (sign << 7) | fraction, i.e. ((w >> 8) & 0x80) | (w & 0x7F);
 *  - chunks of 32768 elements (64 KiB of BF16 output), each with its start
 *    bit; the N bits of a chunk are cut into 512 windows as evenly as
 *    integers allow (window i starts floor(i * N / 512) bits after the
 *    chunk's first bit), with one 16-bit entry per window: the number of
 *    codes that start in it (at most 1536, as a window has at most
 *    ceil(32768 * 24 / 512) bits, so 11 bits) and the offset of the first of
 *    them from the window's first bit (under 24, so 5 bits): a smaller block
 *    index, in the spirit of the df11pack page's experimental 8-bit index
 *    ("Beyond the official format").
 *
 * Container version 4 (all integers little-endian, sections 256-byte aligned):
 *   header, 512 bytes:
 *     0  char[8] magic "DF11HIPC"     8  u32 version (4)   12 u32 flags
 *    16  u64 n_elems                 24  u32 ndim          28 u32 chunk_elems
 *    32  u64 dims[8]                 96  u8 max_code_len   97 u8 reserved
 *    98  u16 windows                100  u32 n_chunks     104 u64 total_bits
 *   112  u64 off_chunk_index        120  u64 off_windows  128 u64 reserved
 *   136  u64 off_stream             144  u64 stream_bytes 152 u64 off_raw
 *   160  u64 raw_bytes              168  u64 total_bytes  176 u8 sha256[32]
 *   208  u8 code_len[256]           464  reserved[48]
 *   chunk index: (n_chunks+1) x {u64 start_bit, u64 out_elem}, last = sentinel
 *                {total_bits, n_elems}
 *   windows:     n_chunks x 512 x u16: cnt | (gap << 11), cnt = codes that
 *                start in the window, gap = offset of the first of them from
 *                the window's first bit; 0 for a window with no code start
 *   stream:      ceil(total_bits/8) bytes rounded up to 16, plus 16 zero bytes
 *   raw:         n_elems bytes rounded up to 16
 *   flags: bit 0 set = sha256 holds the SHA-256 (FIPS 180-4) of the source
 *   tensor's bytes, each word least significant byte first (the df11pack
 *   page, "Beyond the official format": a per-tensor SHA-256 in the header
 *   lets a verify find corruption without the source); clear = sha256 is
 *   zero.  No other flag bit is defined.
 *   Every byte not named above is zero.
 */
#include "df11_oracle.h"

#include <stdlib.h>
#include <string.h>

#define CAP 24
#define CHUNK 32768u
#define WINDOWS 512
#define VERSION 4
#define HDR 512u

/* ------------------------------------------------------------------ */
/* little-endian field access                                          */
/* ------------------------------------------------------------------ */
static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) { uint32_t v = 0; for (int i = 3; i >= 0; i--) v = (v << 8) | p[i]; return v; }
static uint64_t get_u64(const uint8_t *p) { uint64_t v = 0; for (int i = 7; i >= 0; i--) v = (v << 8) | p[i]; return v; }
static uint64_t align256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }
static uint64_t round16(uint64_t x) { return (x + 15u) & ~(uint64_t)15u; }

/* ------------------------------------------------------------------ */
/* The split of one BF16 word (mlx-dfloat, 16-bit weight diagram).     */
/* ------------------------------------------------------------------ */
static unsigned exponent_of(uint16_t w) { return (w >> 7) & 0xFFu; }
static unsigned raw_of(uint16_t w) { return ((w >> 8) & 0x80u) | (w & 0x7Fu); }
static uint16_t join(unsigned e, unsigned r) {
    return (uint16_t)(((r & 0x80u) << 8) | ((e & 0xFFu) << 7) | (r & 0x7Fu));
}

/* ------------------------------------------------------------------ */
/* Package-merge: optimal prefix code with lengths <= cap.             */
/* An item is a weight and, for every symbol, how many times the       */
/* symbol's leaf occurs inside the item.                               */
/* ------------------------------------------------------------------ */
typedef struct {
    uint64_t weight;
    int is_leaf;
    uint8_t count[256];
} item_t;

int oracle_code_lengths(const uint64_t *freq, int cap, uint8_t *len) {
    if (!freq || !len || cap < 1 || cap > 32) return ORACLE_E_ARG;
    memset(len, 0, 256);

    int sym[256], n = 0;
    for (int s = 0; s < 256; s++)
        if (freq[s] > 0) sym[n++] = s;
    if (n == 0) return ORACLE_OK;
    if (n == 1) { len[sym[0]] = 1; return ORACLE_OK; }
    if (cap < 9 && n > (1 << cap)) return ORACLE_E_ARG; /* no code of n words fits */

    /* leaves sorted by (frequency, symbol): insertion sort, n <= 256 */
    for (int i = 1; i < n; i++) {
        int s = sym[i], j = i - 1;
        while (j >= 0 && (freq[sym[j]] > freq[s] || (freq[sym[j]] == freq[s] && sym[j] > s))) {
            sym[j + 1] = sym[j];
            j--;
        }
        sym[j + 1] = s;
    }
    item_t *leaves = calloc((size_t)n, sizeof(item_t));
    item_t *prev = calloc((size_t)2 * n, sizeof(item_t));
    item_t *cur = calloc((size_t)2 * n, sizeof(item_t));
    if (!leaves || !prev || !cur) { free(leaves); free(prev); free(cur); return ORACLE_E_ARG; }
    for (int i = 0; i < n; i++) {
        leaves[i].weight = freq[sym[i]];
        leaves[i].is_leaf = 1;
        leaves[i].count[sym[i]] = 1;
    }

    /* deepest level: the leaves alone */
    int nprev = n;
    memcpy(prev, leaves, sizeof(item_t) * (size_t)n);

    /* each shallower level: merge the leaves with the packages (pairs) of
     * the level below; on equal weight the leaf comes first */
    for (int level = cap - 1; level >= 1; level--) {
        int npk = nprev / 2, il = 0, ip = 0, nc = 0;
        while (il < n || ip < npk) {
            item_t pk;
            int have_pk = ip < npk;
            if (have_pk) {
                const item_t *a = &prev[2 * ip], *b = &prev[2 * ip + 1];
                pk.weight = a->weight + b->weight;
                pk.is_leaf = 0;
                for (int s = 0; s < 256; s++) pk.count[s] = (uint8_t)(a->count[s] + b->count[s]);
            }
            if (il < n && (!have_pk || leaves[il].weight <= pk.weight)) {
                cur[nc++] = leaves[il++];
            } else {
                cur[nc++] = pk;
                ip++;
            }
        }
        item_t *t = prev; prev = cur; cur = t;
        nprev = nc;
    }

    /* the 2n-2 lightest items of the top level; a symbol's code length is
     * the number of times its leaf occurs in them */
    unsigned total[256];
    memset(total, 0, sizeof(total));
    for (int i = 0; i < 2 * n - 2; i++)
        for (int s = 0; s < 256; s++) total[s] += prev[i].count[s];
    for (int s = 0; s < 256; s++) len[s] = (uint8_t)total[s];

    free(leaves); free(prev); free(cur);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Canonical code values (deflate construction, RFC 1951 3.2.2).      */
/* ------------------------------------------------------------------ */
static int sorted_by_length(const uint8_t *len, int *order) {
    int n = 0;
    for (int l = 1; l <= 32; l++)
        for (int s = 0; s < 256; s++)
            if (len[s] == l) order[n++] = s;
    return n;
}

int oracle_canonical_codes(const uint8_t *len, uint32_t *code) {
    if (!len || !code) return ORACLE_E_ARG;
    memset(code, 0, 256 * sizeof(uint32_t));
    int order[256];
    int n = sorted_by_length(len, order);
    uint32_t c = 0;
    for (int i = 0; i < n; i++) {
        if (i > 0) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
        code[order[i]] = c;
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* SHA-256 (FIPS 180-4, sections 4.1.2, 4.2.2, 5.1.1, 5.3.3, 6.2),      */
/* one byte at a time                                                  */
/* ------------------------------------------------------------------ */
/* floor(x^(1/k)), k = 2 or 3, of x < 2^105, by bisection */
static uint64_t iroot(unsigned __int128 x, int k) {
    uint64_t lo = 0, hi = (uint64_t)1 << 36;
    while (lo < hi) {
        uint64_t mid = lo + (hi - lo + 1) / 2;
        unsigned __int128 p = (unsigned __int128)mid * mid;
        if (k == 3) p *= mid;
        if (p <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* The first n primes. */
static void first_primes(int n, uint32_t *p) {
    int found = 0;
    for (uint32_t c = 2; found < n; c++) {
        int prime = 1;
        for (uint32_t d = 2; d * d <= c; d++) if (c % d == 0) { prime = 0; break; }
        if (prime) p[found++] = c;
    }
}

typedef struct {
    uint32_t k[64];     /* first 32 fraction bits of the cube roots of the first 64 primes */
    uint32_t h[8];      /* the hash value; starts at the first 32 fraction bits of the
                           square roots of the first 8 primes */
    uint8_t block[64];
    unsigned fill;
    uint64_t length;    /* message bytes so far */
} sha256_t;

static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

static void sha256_init(sha256_t *S) {
    uint32_t p[64];
    first_primes(64, p);
    /* floor(2^32 * r) mod 2^32 for r = p^(1/k): floor((p * 2^(32k))^(1/k)) */
    for (int i = 0; i < 64; i++) S->k[i] = (uint32_t)iroot((unsigned __int128)p[i] << 96, 3);
    for (int i = 0; i < 8; i++) S->h[i] = (uint32_t)iroot((unsigned __int128)p[i] << 64, 2);
    S->fill = 0;
    S->length = 0;
}

/* One 512-bit block into the hash value (the compression function). */
static void sha256_block(sha256_t *S) {
    uint32_t w[64];
    for (int t = 0; t < 16; t++)
        w[t] = ((uint32_t)S->block[4 * t] << 24) | ((uint32_t)S->block[4 * t + 1] << 16) |
               ((uint32_t)S->block[4 * t + 2] << 8) | S->block[4 * t + 3];
    for (int t = 16; t < 64; t++) {
        uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
        uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
        w[t] = s1 + w[t - 7] + s0 + w[t - 16];
    }
    uint32_t a = S->h[0], b = S->h[1], c = S->h[2], d = S->h[3];
    uint32_t e = S->h[4], f = S->h[5], g = S->h[6], h = S->h[7];
    for (int t = 0; t < 64; t++) {
        uint32_t big1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
        uint32_t ch = (e & f) ^ (~e & g);
        uint32_t t1 = h + big1 + ch + S->k[t] + w[t];
        uint32_t big0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
        uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
        uint32_t t2 = big0 + maj;
        h = g; g = f; f = e; e = d + t1;
        d = c; c = b; b = a; a = t1 + t2;
    }
    S->h[0] += a; S->h[1] += b; S->h[2] += c; S->h[3] += d;
    S->h[4] += e; S->h[5] += f; S->h[6] += g; S->h[7] += h;
}

static void sha256_byte(sha256_t *S, uint8_t x) {
    S->block[S->fill++] = x;
    S->length++;
    if (S->fill == 64) { sha256_block(S); S->fill = 0; }
}

/* Padding: a 1 bit, zeros up to 448 bits mod 512, the bit length (64 bits,
 * big-endian); then the hash value, big-endian. */
static void sha256_final(sha256_t *S, uint8_t out[32]) {
    uint64_t bits = S->length * 8;
    sha256_byte(S, 0x80);
    while (S->fill != 56) sha256_byte(S, 0);
    for (int i = 7; i >= 0; i--) sha256_byte(S, (uint8_t)(bits >> (8 * i)));
    for (int i = 0; i < 8; i++)
        for (int j = 0; j < 4; j++) out[4 * i + j] = (uint8_t)(S->h[i] >> (24 - 8 * j));
}

void oracle_sha256(const uint8_t *msg, uint64_t len, uint8_t out[32]) {
    sha256_t S;
    sha256_init(&S);
    for (uint64_t i = 0; i < len; i++) sha256_byte(&S, msg[i]);
    sha256_final(&S, out);
}

/* SHA-256 of n words as bytes, each word's low byte first. */
static void sha256_words(const uint16_t *w, uint64_t n, uint8_t out[32]) {
    sha256_t S;
    sha256_init(&S);
    for (uint64_t j = 0; j < n; j++) {
        sha256_byte(&S, (uint8_t)(w[j] & 0xFFu));
        sha256_byte(&S, (uint8_t)(w[j] >> 8));
    }
    sha256_final(&S, out);
}

/* ------------------------------------------------------------------ */
/* Encoder                                                             */
/* ------------------------------------------------------------------ */
typedef struct {
    uint64_t n, n_chunks, total_bits;
    uint64_t off_ci, off_win, off_stream, stream_bytes, off_raw, raw_bytes, total;
} layout_t;

static void make_layout(uint64_t n, uint64_t total_bits, layout_t *L) {
    L->n = n;
    L->n_chunks = (n + CHUNK - 1) / CHUNK;
    L->total_bits = total_bits;
    L->off_ci = HDR;
    L->off_win = align256(L->off_ci + (L->n_chunks + 1) * 16);
    L->off_stream = align256(L->off_win + L->n_chunks * WINDOWS * 2);
    L->stream_bytes = round16((total_bits + 7) / 8) + 16;
    L->off_raw = align256(L->off_stream + L->stream_bytes);
    L->raw_bytes = round16(n);
    L->total = L->off_raw + L->raw_bytes;
}

uint64_t oracle_container_bound(uint64_t n) {
    layout_t L;
    make_layout(n, n * CAP, &L);
    return L.total;
}

/* First bit of window i (0 <= i <= 512) of a chunk of N bits, counted from
 * the chunk's first bit: the windows split the N bits as evenly as integers
 * allow (every window has floor(N/512) or ceil(N/512) bits). */
static uint64_t window_edge(uint64_t N, uint64_t i) { return i * N / WINDOWS; }

static void put_bit(uint8_t *stream, uint64_t pos, unsigned bit) {
    if (bit) stream[pos / 8] |= (uint8_t)(0x80u >> (pos % 8));
}
static unsigned get_bit(const uint8_t *stream, uint64_t pos) {
    return (stream[pos / 8] >> (7 - pos % 8)) & 1u;
}

int oracle_encode_flags(const uint16_t *words, uint64_t n, int ndim, const uint64_t *dims, uint32_t flags,
                        uint8_t *out, uint64_t out_cap, uint64_t *out_bytes) {
    if ((!words && n) || !out || !out_bytes || ndim < 0 || ndim > 8 || (ndim && !dims) ||
        (flags & ~(uint32_t)ORACLE_FLAG_SHA256))
        return ORACLE_E_ARG;
    uint64_t prod = 1;
    for (int i = 0; i < ndim; i++) prod *= dims[i];
    if (ndim > 0 && prod != n) return ORACLE_E_ARG;
    if (ndim == 0 && n != 1) return ORACLE_E_ARG;

    /* 1. histogram of the exponent byte */
    uint64_t freq[256];
    memset(freq, 0, sizeof(freq));
    for (uint64_t j = 0; j < n; j++) freq[exponent_of(words[j])]++;

    /* 2. code lengths, 3. canonical codes */
    uint8_t len[256];
    uint32_t code[256];
    oracle_code_lengths(freq, CAP, len);
    oracle_canonical_codes(len, code);

    uint64_t total_bits = 0;
    for (int s = 0; s < 256; s++) total_bits += freq[s] * len[s];

    layout_t L;
    make_layout(n, total_bits, &L);
    if (out_cap < L.total) return ORACLE_E_ARG;
    memset(out, 0, L.total);

    /* header */
    memcpy(out, "DF11HIPC", 8);
    put_u32(out + 8, VERSION);
    put_u32(out + 12, flags);
    if (flags & ORACLE_FLAG_SHA256) sha256_words(words, n, out + 176);
    put_u64(out + 16, n);
    put_u32(out + 24, (uint32_t)ndim);
    put_u32(out + 28, CHUNK);
    for (int i = 0; i < ndim; i++) put_u64(out + 32 + 8 * i, dims[i]);
    out[96] = CAP;
    put_u16(out + 98, WINDOWS);
    put_u32(out + 100, (uint32_t)L.n_chunks);
    put_u64(out + 104, total_bits);
    put_u64(out + 112, L.off_ci);
    put_u64(out + 120, L.off_win);
    put_u64(out + 136, L.off_stream);
    put_u64(out + 144, L.stream_bytes);
    put_u64(out + 152, L.off_raw);
    put_u64(out + 160, L.raw_bytes);
    put_u64(out + 168, L.total);
    memcpy(out + 208, len, 256);

    /* 4. bitstream, most significant bit of each code first, and the chunk
     *    index (start bit of every 32768th code) */
    uint8_t *stream = out + L.off_stream;
    uint64_t pos = 0;
    for (uint64_t j = 0; j < n; j++) {
        if (j % CHUNK == 0) {
            put_u64(out + L.off_ci + (j / CHUNK) * 16, pos);
            put_u64(out + L.off_ci + (j / CHUNK) * 16 + 8, j);
        }
        unsigned e = exponent_of(words[j]);
        for (int b = len[e] - 1; b >= 0; b--) put_bit(stream, pos++, (code[e] >> b) & 1u);
    }
    put_u64(out + L.off_ci + L.n_chunks * 16, total_bits);
    put_u64(out + L.off_ci + L.n_chunks * 16 + 8, n);

    /* 5. window index: the chunk's bits cut into 512 windows (window_edge);
     *    per window the number of code starts and the offset of the first
     *    of them from the window's first bit */
    for (uint64_t c = 0; c < L.n_chunks; c++) {
        uint64_t b0 = get_u64(out + L.off_ci + c * 16);
        uint64_t b1 = get_u64(out + L.off_ci + (c + 1) * 16);
        unsigned cnt[WINDOWS], gap[WINDOWS];
        memset(cnt, 0, sizeof(cnt));
        memset(gap, 0, sizeof(gap));
        uint64_t p = b0;
        int win = 0;
        uint64_t j_end = (c + 1) * CHUNK < n ? (c + 1) * CHUNK : n;
        for (uint64_t j = c * CHUNK; j < j_end; j++) {
            /* the window holding bit p: the last one that starts at or before it */
            while (win + 1 < WINDOWS && b0 + window_edge(b1 - b0, win + 1) <= p) win++;
            if (cnt[win] == 0) gap[win] = (unsigned)(p - (b0 + window_edge(b1 - b0, win)));
            cnt[win]++;
            p += len[exponent_of(words[j])];
        }
        for (int i = 0; i < WINDOWS; i++)
            put_u16(out + L.off_win + (c * WINDOWS + i) * 2, (uint16_t)(cnt[i] | (gap[i] << 11)));
    }

    /* 6. raw bytes: sign and fraction, as is */
    for (uint64_t j = 0; j < n; j++) out[L.off_raw + j] = (uint8_t)raw_of(words[j]);

    *out_bytes = L.total;
    return ORACLE_OK;
}

int oracle_encode(const uint16_t *words, uint64_t n, int ndim, const uint64_t *dims,
                  uint8_t *out, uint64_t out_cap, uint64_t *out_bytes) {
    return oracle_encode_flags(words, n, ndim, dims, 0, out, out_cap, out_bytes);
}

/* ------------------------------------------------------------------ */
/* Header parsing shared by the decoders and the checker               */
/* ------------------------------------------------------------------ */
typedef struct {
    layout_t L;
    uint8_t len[256];
    /* canonical decode table, one bit at a time */
    uint32_t first[CAP + 1];   /* code value of the first symbol of each length */
    uint32_t count[CAP + 1];   /* how many symbols have each length */
    uint32_t offset[CAP + 1];  /* index of that first symbol in `order` */
    int order[256];
} parsed_t;

static int parse(const uint8_t *c, uint64_t bytes, parsed_t *P) {
    if (!c || bytes < HDR) return ORACLE_E_FORMAT;
    if (memcmp(c, "DF11HIPC", 8) != 0 || get_u32(c + 8) != VERSION) return ORACLE_E_FORMAT;
    uint64_t n = get_u64(c + 16);
    uint64_t total_bits = get_u64(c + 104);
    make_layout(n, total_bits, &P->L);
    const layout_t *L = &P->L;
    if (get_u32(c + 28) != CHUNK || c[96] != CAP || get_u16(c + 98) != WINDOWS) return ORACLE_E_FORMAT;
    if (get_u32(c + 100) != L->n_chunks) return ORACLE_E_FORMAT;
    if (get_u64(c + 112) != L->off_ci || get_u64(c + 120) != L->off_win ||
        get_u64(c + 128) != 0 || get_u64(c + 136) != L->off_stream ||
        get_u64(c + 144) != L->stream_bytes || get_u64(c + 152) != L->off_raw ||
        get_u64(c + 160) != L->raw_bytes || get_u64(c + 168) != L->total)
        return ORACLE_E_FORMAT;
    if (bytes < L->total) return ORACLE_E_FORMAT;
    memcpy(P->len, c + 208, 256);
    for (int s = 0; s < 256; s++)
        if (P->len[s] > CAP) return ORACLE_E_FORMAT;

    uint32_t code[256];
    oracle_canonical_codes(P->len, code);
    int n_sym = sorted_by_length(P->len, P->order);
    memset(P->first, 0, sizeof(P->first));
    memset(P->count, 0, sizeof(P->count));
    memset(P->offset, 0, sizeof(P->offset));
    for (int i = n_sym - 1; i >= 0; i--) {
        int l = P->len[P->order[i]];
        P->first[l] = code[P->order[i]];
        P->offset[l] = (uint32_t)i;
        P->count[l]++;
    }
    return ORACLE_OK;
}

/* Read one code starting at *pos, one bit at a time.  Returns the symbol or
 * a negative error. */
static int read_code(const parsed_t *P, const uint8_t *stream, uint64_t *pos) {
    uint32_t v = 0;
    for (int k = 1; k <= CAP; k++) {
        if (*pos >= P->L.total_bits) return -ORACLE_E_TRUNCATED;
        v = (v << 1) | get_bit(stream, (*pos)++);
        if (P->count[k] && v >= P->first[k] && v - P->first[k] < P->count[k])
            return P->order[P->offset[k] + (v - P->first[k])];
    }
    return -ORACLE_E_CORRUPT;
}

int oracle_decode(const uint8_t *c, uint64_t bytes, uint16_t *out, uint64_t n) {
    parsed_t P;
    int st = parse(c, bytes, &P);
    if (st) return st;
    if (n != P.L.n || (!out && n)) return ORACLE_E_ARG;
    const uint8_t *stream = c + P.L.off_stream;
    uint64_t pos = 0;
    for (uint64_t j = 0; j < n; j++) {
        int e = read_code(&P, stream, &pos);
        if (e < 0) return -e;
        out[j] = join((unsigned)e, c[P.L.off_raw + j]);
    }
    return pos == P.L.total_bits ? ORACLE_OK : ORACLE_E_CORRUPT;
}

int oracle_decode_chunk(const uint8_t *c, uint64_t bytes, uint64_t chunk, uint16_t *out) {
    parsed_t P;
    int st = parse(c, bytes, &P);
    if (st) return st;
    if (chunk >= P.L.n_chunks || !out) return ORACLE_E_ARG;
    const uint8_t *stream = c + P.L.off_stream;
    uint64_t pos = get_u64(c + P.L.off_ci + chunk * 16);
    uint64_t j0 = get_u64(c + P.L.off_ci + chunk * 16 + 8);
    uint64_t j1 = get_u64(c + P.L.off_ci + (chunk + 1) * 16 + 8);
    if (j0 > j1 || j1 > P.L.n) return ORACLE_E_FORMAT;
    for (uint64_t j = j0; j < j1; j++) {
        int e = read_code(&P, stream, &pos);
        if (e < 0) return -e;
        out[j - j0] = join((unsigned)e, c[P.L.off_raw + j]);
    }
    return pos == get_u64(c + P.L.off_ci + (chunk + 1) * 16) ? ORACLE_OK : ORACLE_E_CORRUPT;
}

int oracle_decode_window(const uint8_t *c, uint64_t bytes, uint64_t chunk, int win,
                       uint16_t *out, uint64_t *n_out, uint64_t *end_bit) {
    parsed_t P;
    int st = parse(c, bytes, &P);
    if (st) return st;
    if (chunk >= P.L.n_chunks || win < 0 || win >= WINDOWS || !n_out || !end_bit)
        return ORACLE_E_ARG;
    const uint8_t *stream = c + P.L.off_stream;
    uint64_t b0 = get_u64(c + P.L.off_ci + chunk * 16);
    uint64_t b1 = get_u64(c + P.L.off_ci + (chunk + 1) * 16);
    uint64_t ws = b0 + window_edge(b1 - b0, (uint64_t)win);
    const uint8_t *wins = c + P.L.off_win + chunk * WINDOWS * 2;
    unsigned ent = get_u16(wins + 2 * win);
    unsigned cnt = ent & 0x7FFu, gap = ent >> 11;
    /* output position of this window's first code: codes of earlier windows */
    uint64_t before = 0;
    for (int i = 0; i < win; i++) before += get_u16(wins + 2 * i) & 0x7FFu;
    uint64_t j0 = get_u64(c + P.L.off_ci + chunk * 16 + 8) + before;
    *n_out = cnt;
    if (cnt == 0) { *end_bit = ws; return gap == 0 ? ORACLE_OK : ORACLE_E_FORMAT; }
    uint64_t pos = ws + gap;
    for (unsigned k = 0; k < cnt; k++) {
        int e = read_code(&P, stream, &pos);
        if (e < 0) return -e;
        if (out) out[k] = join((unsigned)e, c[P.L.off_raw + j0 + k]);
    }
    *end_bit = pos;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Structural check                                                    */
/* ------------------------------------------------------------------ */
int oracle_check(const uint8_t *c, uint64_t bytes) {
    parsed_t P;
    int st = parse(c, bytes, &P);
    if (st) return st;
    const layout_t *L = &P.L;

    /* shape */
    uint32_t ndim = get_u32(c + 24);
    uint32_t flags = get_u32(c + 12);
    if (ndim > 8 || (flags & ~(uint32_t)ORACLE_FLAG_SHA256)) return ORACLE_E_FORMAT;
    uint64_t prod = 1;
    for (uint32_t i = 0; i < ndim; i++) prod *= get_u64(c + 32 + 8 * i);
    if ((ndim > 0 && prod != L->n) || (ndim == 0 && L->n != 1)) return ORACLE_E_FORMAT;

    /* Kraft sum: exactly 1 with two or more symbols, 1/2 with one */
    uint64_t kraft = 0, present = 0;
    for (int s = 0; s < 256; s++)
        if (P.len[s]) { kraft += (uint64_t)1 << (CAP - P.len[s]); present++; }
    if (present == 0 && L->n != 0) return ORACLE_E_FORMAT;
    if (present == 1 && kraft != ((uint64_t)1 << (CAP - 1))) return ORACLE_E_FORMAT;
    if (present >= 2 && kraft != ((uint64_t)1 << CAP)) return ORACLE_E_FORMAT;

    /* re-walk the stream: start bits, sentinel, windows */
    const uint8_t *stream = c + L->off_stream;
    uint64_t pos = 0;
    for (uint64_t ch = 0; ch < L->n_chunks; ch++) {
        const uint8_t *ent = c + L->off_ci + ch * 16;
        if (get_u64(ent) != pos || get_u64(ent + 8) != ch * CHUNK) return ORACLE_E_FORMAT;
        uint64_t b0 = pos;
        uint64_t b1 = get_u64(ent + 16);
        if (b1 < b0 || b1 > L->total_bits) return ORACLE_E_FORMAT;
        unsigned cnt[WINDOWS], gap[WINDOWS];
        memset(cnt, 0, sizeof(cnt));
        memset(gap, 0, sizeof(gap));
        int win = 0;
        uint64_t j_end = (ch + 1) * CHUNK < L->n ? (ch + 1) * CHUNK : L->n;
        for (uint64_t j = ch * CHUNK; j < j_end; j++) {
            if (pos >= b1) return ORACLE_E_FORMAT;
            while (win + 1 < WINDOWS && b0 + window_edge(b1 - b0, win + 1) <= pos) win++;
            if (cnt[win] == 0) gap[win] = (unsigned)(pos - (b0 + window_edge(b1 - b0, win)));
            cnt[win]++;
            int e = read_code(&P, stream, &pos);
            if (e < 0) return -e;
        }
        if (pos != b1) return ORACLE_E_FORMAT;
        for (int i = 0; i < WINDOWS; i++)
            if (get_u16(c + L->off_win + (ch * WINDOWS + i) * 2) != (cnt[i] | (gap[i] << 11)))
                return ORACLE_E_FORMAT;
    }
    if (pos != L->total_bits) return ORACLE_E_FORMAT;
    const uint8_t *sent = c + L->off_ci + L->n_chunks * 16;
    if (get_u64(sent) != L->total_bits || get_u64(sent + 8) != L->n) return ORACLE_E_FORMAT;

    /* every byte the layout does not name is zero (a canonical container) */
    if (!(flags & ORACLE_FLAG_SHA256))
        for (uint64_t i = 176; i < 208; i++) if (c[i]) return ORACLE_E_FORMAT;
    for (uint64_t i = 464; i < HDR; i++) if (c[i]) return ORACLE_E_FORMAT;
    if (c[97]) return ORACLE_E_FORMAT;
    for (uint32_t i = ndim; i < 8; i++) if (get_u64(c + 32 + 8 * i)) return ORACLE_E_FORMAT;
    for (uint64_t b = L->total_bits; b < L->stream_bytes * 8; b++)
        if (get_bit(stream, b)) return ORACLE_E_FORMAT;
    for (uint64_t i = L->n; i < L->raw_bytes; i++) if (c[L->off_raw + i]) return ORACLE_E_FORMAT;
    /* the stored source hash against the hash of the decoded words */
    if (flags & ORACLE_FLAG_SHA256) {
        uint16_t *w = (uint16_t *)malloc((L->n ? L->n : 1) * sizeof(uint16_t));
        if (!w) return ORACLE_E_ARG;
        int st2 = oracle_decode(c, bytes, w, L->n);
        uint8_t h[32];
        if (!st2) sha256_words(w, L->n, h);
        free(w);
        if (st2) return st2;
        if (memcmp(h, c + 176, 32) != 0) return ORACLE_E_CORRUPT;
    }
    return ORACLE_OK;
}
