// SHA-256 (FIPS 180-4) on the host, for the optional per-tensor source hash
// in the container header (df11pack page, "Beyond the official format": a
// SHA-256 per tensor in the header lets a verify find corruption without the
// source).  Whole 64-byte blocks are hashed straight from the input; only
// the padded tail is copied.
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

void compress(uint32_t h[8], const uint8_t *block) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
        w[t] = (uint32_t)block[4 * t] << 24 | (uint32_t)block[4 * t + 1] << 16 | (uint32_t)block[4 * t + 2] << 8 |
               block[4 * t + 3];
    for (int t = 16; t < 64; ++t)
        w[t] = (rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10)) + w[t - 7] +
               (rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3)) + w[t - 16];
    uint32_t v[8];
    memcpy(v, h, sizeof v);
    for (int t = 0; t < 64; ++t) {
        const uint32_t e = v[4], a = v[0];
        const uint32_t t1 = v[7] + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & v[5]) ^ (~e & v[6])) +
                            kSha.k[t] + w[t];
        const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & v[1]) ^ (a & v[2]) ^ (v[1] & v[2]));
        memmove(v + 1, v, 7 * sizeof(uint32_t));
        v[4] += t1;
        v[0] = t1 + t2;
    }
    for (int i = 0; i < 8; ++i) h[i] += v[i];
}

}  // namespace

void sha256(const void *data, uint64_t bytes, uint8_t out[32]) {
    const uint8_t *p = static_cast<const uint8_t *>(data);
    uint32_t h[8];
    memcpy(h, kSha.h0, sizeof h);
    const uint64_t whole = bytes / 64;
    for (uint64_t b = 0; b < whole; ++b) compress(h, p + 64 * b);
    // the tail, a 1 bit, zeros and the message length in bits, big-endian
    uint8_t tail[128] = {};
    const uint64_t rest = bytes - 64 * whole;
    memcpy(tail, p + 64 * whole, rest);
    tail[rest] = 0x80;
    const uint64_t tail_len = rest + 9 <= 64 ? 64 : 128;
    const uint64_t bits = bytes * 8;
    for (int i = 0; i < 8; ++i) tail[tail_len - 1 - i] = (uint8_t)(bits >> (8 * i));
    for (uint64_t b = 0; b < tail_len; b += 64) compress(h, tail + b);
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

}  // namespace df11

extern "C" void df11_sha256(const void *data, uint64_t bytes, uint8_t *digest) {
    df11::sha256(data, bytes, digest);
}
