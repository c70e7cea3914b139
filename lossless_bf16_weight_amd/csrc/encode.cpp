// libdf11 encoder: BF16 words -> version-4 container (layout in include/df11.h),
// multi-threaded on the host.
//
// Method: mlx-dfloat project page, introduction and 16-bit weight diagram --
// the exponent byte of every weight gets a variable-length prefix code and
// the sign + 7-bit fraction are kept as one raw byte.  The code is the
// optimal prefix code with lengths <= 24 (package-merge, Larmore and
// Hirschberg 1990; leaves ordered by (frequency, symbol), a leaf before a
// package of equal weight), with canonical code values (deflate counting
// construction, RFC 1951 3.2.2).  df11pack's page (introduction, "Measured")
// is the context for doing this fast on CPU cores.
//
// Parallel plan: histogram per thread slice; one chunk per task for the bit
// counts, the packing and the window index (chunks start at known bit offsets
// once the per-chunk bit counts are summed); raw bytes per slice.  The output
// does not depend on the thread count.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

#include "df11_internal.hpp"

using namespace df11;

namespace {

template <class F>
void parallel_for(uint64_t n_tasks, int threads, F &&fn) {
    if (n_tasks == 0) return;
    const int T = (int)std::min<uint64_t>((uint64_t)threads, n_tasks);
    if (T <= 1) {
        for (uint64_t i = 0; i < n_tasks; ++i) fn(i);
        return;
    }
    std::atomic<uint64_t> next{0};
    std::vector<std::thread> pool;
    pool.reserve(T);
    for (int t = 0; t < T; ++t)
        pool.emplace_back([&] {
            for (uint64_t i; (i = next.fetch_add(1)) < n_tasks;) fn(i);
        });
    for (auto &th : pool) th.join();
}

inline uint64_t up256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
inline uint64_t up16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
inline void wr16(uint8_t *p, uint16_t v) { memcpy(p, &v, 2); }
inline void wr32(uint8_t *p, uint32_t v) { memcpy(p, &v, 4); }
inline void wr64(uint8_t *p, uint64_t v) { memcpy(p, &v, 8); }

// Package-merge by levels.  Level 0's list is the leaves (symbols) by
// weight; level d's list merges the leaves with the packages of level d-1
// (package i pairs items 2i and 2i+1 of that list), a leaf before a package
// of equal weight.  The lengths follow by counting, so each level keeps only
// which of its items are packages: the 2n-2 lightest items of the top level
// are selected, a selected prefix of level d holding p packages selects the
// first 2p items of level d-1, and a symbol's length is the number of levels
// whose selected prefix holds its leaf (the selected leaves of a level are
// always the lightest ones).  Fixed-size arrays only: nothing is allocated.
void package_merge(const uint64_t *freq, int cap, uint8_t *len) {
    memset(len, 0, 256);
    int sym[256], n = 0;
    for (int s = 0; s < 256; ++s)
        if (freq[s]) sym[n++] = s;
    if (n == 0) return;
    if (n == 1) { len[sym[0]] = 1; return; }
    // by (frequency, symbol): a total order, so the result is the stable sort
    std::sort(sym, sym + n, [&](int a, int b) { return freq[a] < freq[b] || (freq[a] == freq[b] && a < b); });

    // a level's list has at most n + (2n - 2) / 2 < 512 items
    static_assert(kMaxLen <= 32, "levels");
    uint64_t wbuf[2][512];
    uint8_t is_pkg[kMaxLen][512];
    int count[kMaxLen];
    uint64_t *below = wbuf[0], *cur = wbuf[1];
    for (int i = 0; i < n; ++i) {
        below[i] = freq[sym[i]];
        is_pkg[0][i] = 0;
    }
    count[0] = n;
    for (int d = 1; d < cap; ++d) {
        int il = 0, ip = 0, k = 0;
        const int np = count[d - 1] / 2;
        while (il < n || ip < np) {
            const uint64_t pw = ip < np ? below[2 * ip] + below[2 * ip + 1] : 0;
            const bool take_leaf = ip >= np || (il < n && freq[sym[il]] <= pw);
            if (take_leaf) {
                cur[k] = freq[sym[il++]];
                is_pkg[d][k] = 0;
            } else {
                cur[k] = pw;
                is_pkg[d][k] = 1;
                ++ip;
            }
            ++k;
        }
        count[d] = k;
        std::swap(below, cur);
    }
    int m = 2 * n - 2;
    for (int d = cap - 1; d >= 0; --d) {
        int leaves = 0, pkgs = 0;
        for (int i = 0; i < m; ++i) is_pkg[d][i] ? ++pkgs : ++leaves;
        for (int i = 0; i < leaves; ++i) len[sym[i]]++;
        m = 2 * pkgs;
    }
}

void canonical_codes(const uint8_t *len, uint32_t *code) {
    uint32_t bl_count[kMaxLen + 1] = {}, next_code[kMaxLen + 2] = {};
    for (int s = 0; s < 256; ++s)
        if (len[s]) bl_count[len[s]]++;
    uint32_t c = 0;
    for (int bits = 1; bits <= kMaxLen; ++bits) {
        c = (c + bl_count[bits - 1]) << 1;
        next_code[bits] = c;
    }
    for (int s = 0; s < 256; ++s) code[s] = len[s] ? next_code[len[s]]++ : 0;
}

}  // namespace

namespace df11 {

void build_code(const uint64_t *freq, uint8_t *len, uint32_t *code) {
    package_merge(freq, kMaxLen, len);
    canonical_codes(len, code);
}

EncodeLayout encode_layout(uint64_t n, uint64_t total_bits) {
    EncodeLayout L;
    L.n_chunks = (n + kChunk - 1) / kChunk;
    L.total_bits = total_bits;
    L.off_ci = kHeader;
    L.off_win = up256(L.off_ci + (L.n_chunks + 1) * 16);
    L.off_stream = up256(L.off_win + L.n_chunks * kWindows * 2);
    L.stream_bytes = up16((total_bits + 7) / 8) + 16;
    L.off_raw = up256(L.off_stream + L.stream_bytes);
    L.raw_bytes = up16(n);
    L.total = L.off_raw + L.raw_bytes;
    return L;
}

void write_header(uint8_t *out, uint64_t n, int ndim, const uint64_t *dims, const EncodeLayout &L,
                  const uint8_t *len) {
    memset(out, 0, kHeader);
    memcpy(out, "DF11HIPC", 8);
    wr32(out + 8, kVersion);
    wr64(out + 16, n);
    wr32(out + 24, (uint32_t)ndim);
    wr32(out + 28, kChunk);
    for (int i = 0; i < ndim; ++i) wr64(out + 32 + 8 * i, dims[i]);
    out[96] = kMaxLen;
    wr16(out + 98, kWindows);
    wr32(out + 100, (uint32_t)L.n_chunks);
    wr64(out + 104, L.total_bits);
    wr64(out + 112, L.off_ci);
    wr64(out + 120, L.off_win);
    wr64(out + 136, L.off_stream);
    wr64(out + 144, L.stream_bytes);
    wr64(out + 152, L.off_raw);
    wr64(out + 160, L.raw_bytes);
    wr64(out + 168, L.total);
    memcpy(out + 208, len, 256);
}

}  // namespace df11

extern "C" df11_status df11_encode_ex(const uint16_t *w, uint64_t n, int ndim, const uint64_t *dims, uint32_t flags,
                                      void *out_v, uint64_t out_cap, uint64_t *out_bytes, int threads) {
    uint8_t *out = (uint8_t *)out_v;
    if ((!w && n) || !out || !out_bytes || ndim < 0 || ndim > 8 || (ndim && !dims) || (flags & ~DF11_FLAG_SHA256))
        return DF11_E_ARG;
    uint64_t prod = 1;
    for (int i = 0; i < ndim; ++i) prod *= dims[i];
    if ((ndim && prod != n) || (!ndim && n != 1)) return DF11_E_ARG;
    if (n > (uint64_t(1) << 46)) return DF11_E_UNSUPPORTED;
    if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
    // the source hash, on a thread of its own while the rest is encoded
    uint8_t digest[32] = {};
    std::thread hasher;
    if (flags & DF11_FLAG_SHA256) hasher = std::thread([&] { sha256(w, 2 * n, digest); });
    struct Join {
        std::thread &t;
        ~Join() { if (t.joinable()) t.join(); }
    } join{hasher};

    // 1. exponent histogram
    const uint64_t n_slices = std::max<uint64_t>(1, std::min<uint64_t>((n + (1 << 20) - 1) >> 20, 4096));
    std::vector<uint64_t> part(n_slices * 256, 0);
    parallel_for(n_slices, threads, [&](uint64_t s) {
        const uint64_t lo = n * s / n_slices, hi = n * (s + 1) / n_slices;
        uint64_t *h = &part[s * 256];
        for (uint64_t j = lo; j < hi; ++j) h[(w[j] >> 7) & 0xFF]++;
    });
    uint64_t freq[256] = {};
    for (uint64_t s = 0; s < n_slices; ++s)
        for (int e = 0; e < 256; ++e) freq[e] += part[s * 256 + e];

    // 2. lengths, 3. canonical codes
    uint8_t len[256];
    uint32_t code[256];
    build_code(freq, len, code);

    // 4. per-chunk bit counts and start bits
    const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
    std::vector<uint64_t> start(n_chunks + 1, 0);
    parallel_for(n_chunks, threads, [&](uint64_t c) {
        const uint64_t lo = c * kChunk, hi = std::min<uint64_t>(n, lo + kChunk);
        uint64_t bits = 0;
        for (uint64_t j = lo; j < hi; ++j) bits += len[(w[j] >> 7) & 0xFF];
        start[c + 1] = bits;
    });
    for (uint64_t c = 0; c < n_chunks; ++c) start[c + 1] += start[c];
    const uint64_t total_bits = start[n_chunks];

    // layout
    const EncodeLayout EL = encode_layout(n, total_bits);
    const uint64_t off_ci = EL.off_ci, off_win = EL.off_win, off_stream = EL.off_stream;
    const uint64_t off_raw = EL.off_raw, total = EL.total;
    if (out_cap < total) return DF11_E_ARG;

    // zero everything (padding and reserved bytes stay zero)
    const uint64_t zslices = std::max<uint64_t>(1, total >> 24);
    parallel_for(zslices, threads, [&](uint64_t s) {
        const uint64_t lo = total * s / zslices, hi = total * (s + 1) / zslices;
        memset(out + lo, 0, hi - lo);
    });

    write_header(out, n, ndim, dims, EL, len);
    for (uint64_t c = 0; c <= n_chunks; ++c) {
        wr64(out + off_ci + c * 16, start[c]);
        wr64(out + off_ci + c * 16 + 8, std::min<uint64_t>(c * kChunk, n));
    }

    // 5. pack each chunk's codes and build its window index
    uint8_t *stream = out + off_stream;
    parallel_for(n_chunks, threads, [&](uint64_t c) {
        thread_local std::vector<uint8_t> buf;
        const uint64_t lo = c * kChunk, hi = std::min<uint64_t>(n, lo + kChunk);
        const uint64_t b0 = start[c], b1 = start[c + 1];
        const uint32_t nbits = (uint32_t)(b1 - b0);
        const unsigned head = (unsigned)(b0 & 7);
        const uint64_t nbytes = (head + (b1 - b0) + 7) / 8;
        buf.assign(nbytes + 8, 0);
        unsigned cnt[kWindows] = {};
        unsigned gap[kWindows] = {};
        uint64_t acc = 0;   // pending bits, right-aligned
        unsigned nacc = head;
        uint64_t at = 0, pos = 0;   // output byte, chunk-relative bit position
        unsigned win = 0;           // the window holding bit pos
        for (uint64_t j = lo; j < hi; ++j) {
            const unsigned e = (w[j] >> 7) & 0xFF;
            while (win + 1 < (unsigned)kWindows && window_edge(nbits, win + 1) <= pos) ++win;
            if (cnt[win]++ == 0) gap[win] = (unsigned)(pos - window_edge(nbits, win));
            acc = (acc << len[e]) | code[e];
            nacc += len[e];
            pos += len[e];
            while (nacc >= 8) {
                nacc -= 8;
                buf[at++] = (uint8_t)(acc >> nacc);
            }
        }
        if (nacc) buf[at++] = (uint8_t)(acc << (8 - nacc));
        // bytes shared with the neighbouring chunks are merged with an OR
        const uint64_t first = b0 / 8;
        for (uint64_t i = 0; i < at; ++i) {
            const bool shared = (i == 0 && head) || (i + 1 == at && ((head + (b1 - b0)) & 7));
            if (shared) __atomic_fetch_or(&stream[first + i], buf[i], __ATOMIC_RELAXED);
            else stream[first + i] = buf[i];
        }
        // (a window has at most 1536 bits, so cnt fits 11 bits; gap < 24)
        for (int i = 0; i < kWindows; ++i)
            wr16(out + off_win + (c * kWindows + i) * 2, (uint16_t)(cnt[i] | (gap[i] << kWinGapShift)));
    });

    // 6. raw bytes
    parallel_for(n_slices, threads, [&](uint64_t s) {
        const uint64_t lo = n * s / n_slices, hi = n * (s + 1) / n_slices;
        uint8_t *r = out + off_raw;
        for (uint64_t j = lo; j < hi; ++j) r[j] = (uint8_t)(((w[j] >> 8) & 0x80) | (w[j] & 0x7F));
    });

    if (hasher.joinable()) hasher.join();
    if (flags & DF11_FLAG_SHA256) {
        wr32(out + 12, flags);
        memcpy(out + 176, digest, 32);
    }
    *out_bytes = total;
    return DF11_OK;
}

extern "C" df11_status df11_encode(const uint16_t *w, uint64_t n, int ndim, const uint64_t *dims,
                                   void *out_v, uint64_t out_cap, uint64_t *out_bytes, int threads) {
    return df11_encode_ex(w, n, ndim, dims, 0, out_v, out_cap, out_bytes, threads);
}
