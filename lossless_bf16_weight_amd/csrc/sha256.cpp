// SHA-256 (FIPS 180-4) on the host, for the optional per-tensor source hash
// in the container header (df11pack page, "Beyond the official format": a
// SHA-256 per tensor in the header lets a verify find corruption without the
// source).  Whole 64-byte blocks are hashed straight from the input; only
// the padded tail is copied.  On x86 processors with the SHA extensions the
// blocks go through them (four rounds per pair of instructions), else
// through portable code.
#include <cpuid.h>
#include <immintrin.h>

#include <cstdlib>
#include <cstring>

#include "df11_internal.hpp"

namespace df11 {

namespace {

// floor(2^32 * frac(r)) of r = p^(1/k), computed as the integer k-th root of
// p * 2^(32 k) by Newton's iteration on 128-bit integers.
uint32_t root_bits(uint32_t p, int k) {
    const unsigned __int128 x = (unsigned __int128)p << (32 * k);
    unsigned __int128 r = (unsigned __int128)1 << (k == 2 ? 36 : 35);   // above the root
    for (;;) {
        const unsigned __int128 y =
            k == 2 ? (r + x / r) / 2 : (2 * r + x / (r * r)) / 3;
        if (y >= r) break;
        r = y;
    }
    return (uint32_t)r;
}

struct Constants {
    uint32_t k[64], h0[8];
    Constants() {
        int found = 0;
        for (uint32_t c = 2; found < 64; ++c) {
            bool prime = true;
            for (uint32_t d = 2; d * d <= c && prime; ++d) prime = c % d != 0;
            if (!prime) continue;
            k[found] = root_bits(c, 3);
            if (found < 8) h0[found] = root_bits(c, 2);
            ++found;
        }
    }
};
const Constants kSha;

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// One round with the working variables named by position: the caller
// rotates the roles instead of moving the values.
inline void round(uint32_t a, uint32_t b, uint32_t c, uint32_t &d, uint32_t e, uint32_t f, uint32_t g,
                  uint32_t &h, uint32_t kw) {
    const uint32_t t1 = h + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + (g ^ (e & (f ^ g))) + kw;
    const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) | (c & (a | b)));
    d += t1;
    h = t1 + t2;
}

void compress(uint32_t hv[8], const uint8_t *block) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
        w[t] = (uint32_t)block[4 * t] << 24 | (uint32_t)block[4 * t + 1] << 16 | (uint32_t)block[4 * t + 2] << 8 |
               block[4 * t + 3];
    for (int t = 16; t < 64; ++t)
        w[t] = (rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10)) + w[t - 7] +
               (rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3)) + w[t - 16];
    uint32_t a = hv[0], b = hv[1], c = hv[2], d = hv[3], e = hv[4], f = hv[5], g = hv[6], h = hv[7];
    for (int t = 0; t < 64; t += 8) {
        round(a, b, c, d, e, f, g, h, kSha.k[t] + w[t]);
        round(h, a, b, c, d, e, f, g, kSha.k[t + 1] + w[t + 1]);
        round(g, h, a, b, c, d, e, f, kSha.k[t + 2] + w[t + 2]);
        round(f, g, h, a, b, c, d, e, kSha.k[t + 3] + w[t + 3]);
        round(e, f, g, h, a, b, c, d, kSha.k[t + 4] + w[t + 4]);
        round(d, e, f, g, h, a, b, c, kSha.k[t + 5] + w[t + 5]);
        round(c, d, e, f, g, h, a, b, kSha.k[t + 6] + w[t + 6]);
        round(b, c, d, e, f, g, h, a, kSha.k[t + 7] + w[t + 7]);
    }
    hv[0] += a; hv[1] += b; hv[2] += c; hv[3] += d;
    hv[4] += e; hv[5] += f; hv[6] += g; hv[7] += h;
}

// The same on the SHA extensions.  The state lives in two registers as
// (A, B, E, F) and (C, D, G, H), highest lane first, which is the layout the
// two-round instruction takes; each group of four rounds runs two of them on
// the message words plus constants, and the schedule instructions build the
// next words four at a time.
__attribute__((target("sha,sse4.1,ssse3")))
void compress_sha_ext(uint32_t hv[8], const uint8_t *data, uint64_t blocks) {
    const __m128i bswap = _mm_set_epi64x(0x0c0d0e0f08090a0bLL, 0x0405060700010203LL);
    const __m128i dcba = _mm_shuffle_epi32(_mm_loadu_si128((const __m128i *)hv), 0xB1);
    const __m128i efgh = _mm_shuffle_epi32(_mm_loadu_si128((const __m128i *)(hv + 4)), 0x1B);
    __m128i abef = _mm_alignr_epi8(dcba, efgh, 8);
    __m128i cdgh = _mm_blend_epi16(efgh, dcba, 0xF0);
    for (uint64_t blk = 0; blk < blocks; ++blk, data += 64) {
        const __m128i abef0 = abef, cdgh0 = cdgh;
        __m128i m[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < 4) m[i] = _mm_shuffle_epi8(_mm_loadu_si128((const __m128i *)(data + 16 * i)), bswap);
            __m128i kw = _mm_add_epi32(m[i & 3], _mm_loadu_si128((const __m128i *)(kSha.k + 4 * i)));
            cdgh = _mm_sha256rnds2_epu32(cdgh, abef, kw);   // rounds 4i, 4i+1
            if (i >= 3 && i < 15) {
                // words 4(i+1) .. 4(i+1)+3 from the four groups before
                const __m128i w7 = _mm_alignr_epi8(m[i & 3], m[(i - 1) & 3], 4);
                m[(i + 1) & 3] = _mm_sha256msg2_epu32(_mm_add_epi32(m[(i + 1) & 3], w7), m[i & 3]);
            }
            abef = _mm_sha256rnds2_epu32(abef, cdgh, _mm_shuffle_epi32(kw, 0x0E));   // 4i+2, 4i+3
            if (i >= 1 && i < 13) m[(i - 1) & 3] = _mm_sha256msg1_epu32(m[(i - 1) & 3], m[i & 3]);
            // (after two rounds the register called cdgh holds A, B, E, F
            // and after two more it holds C, D, G, H again: the names stay
            // right at every fourth round)
        }
        abef = _mm_add_epi32(abef, abef0);
        cdgh = _mm_add_epi32(cdgh, cdgh0);
    }
    const __m128i feba = _mm_shuffle_epi32(abef, 0x1B);
    const __m128i ghcd = _mm_shuffle_epi32(cdgh, 0xB1);
    _mm_storeu_si128((__m128i *)hv, _mm_blend_epi16(feba, ghcd, 0xF0));
    _mm_storeu_si128((__m128i *)(hv + 4), _mm_alignr_epi8(ghcd, feba, 8));
}

bool have_sha_ext() {
    unsigned a, b, c, d;
    if (!__get_cpuid_count(7, 0, &a, &b, &c, &d)) return false;
    const bool sha = (b >> 29) & 1u;
    if (!__get_cpuid(1, &a, &b, &c, &d)) return false;
    return sha && ((c >> 19) & 1u) && ((c >> 9) & 1u);   // SSE4.1, SSSE3
}
// (DF11_SHA256_PORTABLE set in the environment selects the portable code,
// so that it can be tested on processors with the extensions)
const bool kShaExt = have_sha_ext() && !std::getenv("DF11_SHA256_PORTABLE");

void blocks(uint32_t h[8], const uint8_t *p, uint64_t n) {
    if (kShaExt) {
        compress_sha_ext(h, p, n);
    } else {
        for (uint64_t b = 0; b < n; ++b) compress(h, p + 64 * b);
    }
}

}  // namespace

bool sha256_uses_extensions() { return kShaExt; }

void sha256(const void *data, uint64_t bytes, uint8_t out[32]) {
    const uint8_t *p = static_cast<const uint8_t *>(data);
    uint32_t h[8];
    memcpy(h, kSha.h0, sizeof h);
    const uint64_t whole = bytes / 64;
    blocks(h, p, whole);
    // the tail, a 1 bit, zeros and the message length in bits, big-endian
    uint8_t tail[128] = {};
    const uint64_t rest = bytes - 64 * whole;
    if (rest) memcpy(tail, p + 64 * whole, rest);   // (p may be NULL for an empty message)
    tail[rest] = 0x80;
    const uint64_t tail_len = rest + 9 <= 64 ? 64 : 128;
    const uint64_t bits = bytes * 8;
    for (int i = 0; i < 8; ++i) tail[tail_len - 1 - i] = (uint8_t)(bits >> (8 * i));
    blocks(h, tail, tail_len / 64);
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

}  // namespace df11

extern "C" void df11_sha256(const void *data, uint64_t bytes, uint8_t *digest) {
    df11::sha256(data, bytes, digest);
}
