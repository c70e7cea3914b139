/*
 * Oracle for NF12, the fixed-rate lossless BF16 format.  TEST INFRASTRUCTURE
 * ONLY: the product library never includes, links or calls this file.
 *
 * Plain, slow, obviously-correct C, one element and one bit at a time.
 *
 * Source: the nf12 news page ("Developer open-sources nf12: lossless 12-bit
 * compression for BF16 models"), "How it works" and "Implementation details":
 *  - almost all weights share the top four exponent bits 0111; those bits
 *    are not stored and are put back when decoding;
 *  - weights go in groups of 8; a group whose 8 weights all have them packs
 *    its 16 bytes into 12 (8 x 12 bits: sign, low four exponent bits,
 *    7-bit fraction); any other group is an outlier, flagged, and its 8
 *    original words go to an escape buffer (28 bytes per escaped group: the
 *    12-byte slot it still owns plus its 16 bytes there);
 *  - decoding gives back every word bit for bit.
 *
 * Where the page is silent this file takes one fixed reading:
 *  - a 12-bit code is (sign << 11) | (low four exponent bits << 7) |
 *    fraction; code i of a group occupies bits 12i .. 12i+11 of the group's
 *    12 bytes, bit b being bit b % 8 of byte b / 8;
 *  - outlier flags are a bitmap (bit g % 64 of 64-bit word g / 64 flags
 *    group g), with, per bitmap word, the number of outliers before it, so
 *    that any group finds its escape entry without a walk; an outlier's slot
 *    holds zeros; escape entries are in group order;
 *  - a last, partial group is completed with the word 0x3800 (exponent 0x70,
 *    whose top four bits are 0111), so that only real elements decide
 *    whether it escapes; those words are never decoded.
 *
 * Container (little-endian, sections on 256-byte boundaries):
 *   header, 256 bytes:
 *     0 char[8] "NF12HIPC"   8 u32 version (1)   12 u32 flags (0)
 *    16 u64 n_elems         24 u64 n_groups      32 u64 n_escaped
 *    40 u64 off_slots       48 u64 off_flags     56 u64 off_prefix
 *    64 u64 off_escape      72 u64 total_bytes   80..255 zero
 *   slots:  n_groups x 12 bytes
 *   flags:  ceil(n_groups / 64) x u64
 *   prefix: ceil(n_groups / 64) x u32
 *   escape: n_escaped x 16 bytes
 *   Every byte not named is zero.
 */
#include "nf12_oracle.h"

#include <string.h>

#define NF_HDR 256u
#define NF_VERSION 1u
#define NF_PAD_WORD 0x3800u

static void nput32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void nput64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint32_t nget32(const uint8_t *p) { uint32_t v = 0; for (int i = 3; i >= 0; i--) v = (v << 8) | p[i]; return v; }
static uint64_t nget64(const uint8_t *p) { uint64_t v = 0; for (int i = 7; i >= 0; i--) v = (v << 8) | p[i]; return v; }
static uint64_t nalign256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }

/* The BF16 fields: sign bit 15, exponent bits 14..7, fraction bits 6..0. */
static unsigned sign_of(uint16_t w) { return (w >> 15) & 1u; }
static unsigned exponent_of(uint16_t w) { return (w >> 7) & 0xFFu; }
static unsigned fraction_of(uint16_t w) { return w & 0x7Fu; }

/* A weight fits in 12 bits when the top four of its exponent bits are 0111. */
int oracle_nf12_fits(uint16_t w) { return (exponent_of(w) >> 4) == 0x7u; }

/* (sign << 11) | (low four exponent bits << 7) | fraction */
uint32_t oracle_nf12_code(uint16_t w) {
    return (sign_of(w) << 11) | ((exponent_of(w) & 0xFu) << 7) | fraction_of(w);
}

/* The word back from its code: the dropped bits are 0111. */
uint16_t oracle_nf12_word(uint32_t code) {
    unsigned sign = (code >> 11) & 1u, e = 0x70u | ((code >> 7) & 0xFu), frac = code & 0x7Fu;
    return (uint16_t)((sign << 15) | (e << 7) | frac);
}

typedef struct {
    uint64_t n, n_groups, n_words, n_escaped;
    uint64_t off_slots, off_flags, off_prefix, off_escape, total;
} nf_layout;

static void nf_layout_for(uint64_t n, uint64_t n_escaped, nf_layout *L) {
    L->n = n;
    L->n_groups = (n + 7) / 8;
    L->n_words = (L->n_groups + 63) / 64;
    L->n_escaped = n_escaped;
    L->off_slots = NF_HDR;
    L->off_flags = nalign256(L->off_slots + 12 * L->n_groups);
    L->off_prefix = nalign256(L->off_flags + 8 * L->n_words);
    L->off_escape = nalign256(L->off_prefix + 4 * L->n_words);
    L->total = nalign256(L->off_escape + 16 * n_escaped);
}

uint64_t oracle_nf12_bound(uint64_t n) {
    nf_layout L;
    nf_layout_for(n, (n + 7) / 8, &L);
    return L.total;
}

/* Element i of group g, with the partial last group completed. */
static uint16_t group_word(const uint16_t *w, uint64_t n, uint64_t g, int i) {
    uint64_t j = 8 * g + (uint64_t)i;
    return j < n ? w[j] : (uint16_t)NF_PAD_WORD;
}

static int group_fits(const uint16_t *w, uint64_t n, uint64_t g) {
    for (int i = 0; i < 8; i++)
        if (!oracle_nf12_fits(group_word(w, n, g, i))) return 0;
    return 1;
}

int oracle_nf12_encode(const uint16_t *w, uint64_t n, uint8_t *out, uint64_t cap, uint64_t *out_bytes) {
    if ((!w && n) || !out || !out_bytes) return NF12_ORACLE_E_ARG;
    uint64_t escaped = 0;
    for (uint64_t g = 0; g < (n + 7) / 8; g++) escaped += !group_fits(w, n, g);
    nf_layout L;
    nf_layout_for(n, escaped, &L);
    if (cap < L.total) return NF12_ORACLE_E_ARG;
    memset(out, 0, L.total);
    memcpy(out, "NF12HIPC", 8);
    nput32(out + 8, NF_VERSION);
    nput64(out + 16, L.n);
    nput64(out + 24, L.n_groups);
    nput64(out + 32, L.n_escaped);
    nput64(out + 40, L.off_slots);
    nput64(out + 48, L.off_flags);
    nput64(out + 56, L.off_prefix);
    nput64(out + 64, L.off_escape);
    nput64(out + 72, L.total);
    uint64_t e = 0;
    for (uint64_t g = 0; g < L.n_groups; g++) {
        if (g % 64 == 0) nput32(out + L.off_prefix + 4 * (g / 64), (uint32_t)e);
        if (group_fits(w, n, g)) {
            uint8_t *slot = out + L.off_slots + 12 * g;
            for (int i = 0; i < 8; i++) {
                uint32_t code = oracle_nf12_code(group_word(w, n, g, i));
                for (int b = 0; b < 12; b++)
                    if ((code >> b) & 1u) slot[(12 * i + b) / 8] |= (uint8_t)(1u << ((12 * i + b) % 8));
            }
        } else {
            out[L.off_flags + 8 * (g / 64) + (g % 64) / 8] |= (uint8_t)(1u << (g % 8));
            uint8_t *esc = out + L.off_escape + 16 * e;
            for (int i = 0; i < 8; i++) {
                uint16_t v = group_word(w, n, g, i);
                esc[2 * i] = (uint8_t)v;
                esc[2 * i + 1] = (uint8_t)(v >> 8);
            }
            e++;
        }
    }
    *out_bytes = L.total;
    return NF12_ORACLE_OK;
}

/* Structural check of a whole container: header, layout, flags, prefixes,
 * zero slots of outliers, and zero bytes everywhere else. */
int oracle_nf12_check(const uint8_t *c, uint64_t bytes) {
    if (!c || bytes < NF_HDR) return NF12_ORACLE_E_FORMAT;
    if (memcmp(c, "NF12HIPC", 8) != 0 || nget32(c + 8) != NF_VERSION || nget32(c + 12) != 0)
        return NF12_ORACLE_E_FORMAT;
    uint64_t n = nget64(c + 16), escaped = nget64(c + 32);
    if (n > ((uint64_t)1 << 46) || escaped > (n + 7) / 8) return NF12_ORACLE_E_FORMAT;
    nf_layout L;
    nf_layout_for(n, escaped, &L);
    if (nget64(c + 24) != L.n_groups || nget64(c + 40) != L.off_slots || nget64(c + 48) != L.off_flags ||
        nget64(c + 56) != L.off_prefix || nget64(c + 64) != L.off_escape || nget64(c + 72) != L.total)
        return NF12_ORACLE_E_FORMAT;
    if (bytes < L.total) return NF12_ORACLE_E_FORMAT;
    for (uint64_t i = 80; i < NF_HDR; i++) if (c[i]) return NF12_ORACLE_E_FORMAT;
    uint64_t e = 0;
    for (uint64_t g = 0; g < L.n_groups; g++) {
        if (g % 64 == 0 && nget32(c + L.off_prefix + 4 * (g / 64)) != e) return NF12_ORACLE_E_FORMAT;
        int flag = (c[L.off_flags + 8 * (g / 64) + (g % 64) / 8] >> (g % 8)) & 1;
        if (flag) {
            for (int b = 0; b < 12; b++) if (c[L.off_slots + 12 * g + b]) return NF12_ORACLE_E_FORMAT;
            e++;
        }
    }
    if (e != escaped) return NF12_ORACLE_E_FORMAT;
    /* flag bits past the last group, and every padding byte, are zero */
    for (uint64_t g = L.n_groups; g < 64 * L.n_words; g++)
        if ((c[L.off_flags + 8 * (g / 64) + (g % 64) / 8] >> (g % 8)) & 1) return NF12_ORACLE_E_FORMAT;
    for (uint64_t i = L.off_slots + 12 * L.n_groups; i < L.off_flags; i++) if (c[i]) return NF12_ORACLE_E_FORMAT;
    for (uint64_t i = L.off_flags + 8 * L.n_words; i < L.off_prefix; i++) if (c[i]) return NF12_ORACLE_E_FORMAT;
    for (uint64_t i = L.off_prefix + 4 * L.n_words; i < L.off_escape; i++) if (c[i]) return NF12_ORACLE_E_FORMAT;
    for (uint64_t i = L.off_escape + 16 * L.n_escaped; i < L.total; i++) if (c[i]) return NF12_ORACLE_E_FORMAT;
    return NF12_ORACLE_OK;
}

int oracle_nf12_decode(const uint8_t *c, uint64_t bytes, uint16_t *out, uint64_t n) {
    int st = oracle_nf12_check(c, bytes);
    if (st) return st;
    nf_layout L;
    nf_layout_for(nget64(c + 16), nget64(c + 32), &L);
    if (n != L.n || (!out && n)) return NF12_ORACLE_E_ARG;
    uint64_t e = 0;   /* outliers met so far, counted one group at a time */
    for (uint64_t g = 0; g < L.n_groups; g++) {
        int flag = (c[L.off_flags + 8 * (g / 64) + (g % 64) / 8] >> (g % 8)) & 1;
        for (int i = 0; i < 8; i++) {
            uint64_t j = 8 * g + (uint64_t)i;
            if (j >= n) break;
            if (flag) {
                const uint8_t *esc = c + L.off_escape + 16 * e;
                out[j] = (uint16_t)(esc[2 * i] | (esc[2 * i + 1] << 8));
            } else {
                uint32_t code = 0;
                for (int b = 0; b < 12; b++)
                    code |= (uint32_t)((c[L.off_slots + 12 * g + (12 * i + b) / 8] >> ((12 * i + b) % 8)) & 1u) << b;
                out[j] = oracle_nf12_word(code);
            }
        }
        e += flag;
    }
    return NF12_ORACLE_OK;
}
