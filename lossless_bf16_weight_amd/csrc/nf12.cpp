// NF12, the fixed-rate 12-bit format (nf12 news page, "Developer open-sources
// nf12: lossless 12-bit compression for BF16 models", "How it works" and
// "Implementation details"): host encoder, validation and the decode launch.
// The layout is in include/df11.h.
//
// Parallel plan of the encoder: one task per 64 groups (one bitmap word):
// flags and outlier counts first, then the prefix counts (a serial sum over
// the words), then slots and escape entries.  The output does not depend on
// the thread count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

#include "nf12_internal.hpp"

using namespace df11;

namespace {

template <class F>
void parallel_for(uint64_t n_tasks, int threads, F &&fn) {
    if (n_tasks == 0) return;
    const int T = (int)std::min<uint64_t>((uint64_t)std::max(threads, 1), n_tasks);
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

inline void wr32(uint8_t *p, uint32_t v) { memcpy(p, &v, 4); }
inline void wr64(uint8_t *p, uint64_t v) { memcpy(p, &v, 8); }
inline uint32_t rd32(const uint8_t *p) { uint32_t v; memcpy(&v, p, 4); return v; }
inline uint64_t rd64(const uint8_t *p) { uint64_t v; memcpy(&v, p, 8); return v; }

// A weight fits in 12 bits when the top four of its exponent bits are 0111.
inline bool fits(uint16_t w) { return ((w >> 11) & 0xFu) == 0x7u; }

inline uint16_t group_word(const uint16_t *w, uint64_t n, uint64_t g, int i) {
    const uint64_t j = 8 * g + (uint64_t)i;
    return j < n ? w[j] : kNf12PadWord;
}

inline bool group_fits(const uint16_t *w, uint64_t n, uint64_t g) {
    if (8 * g + 8 <= n) {
        for (int i = 0; i < 8; ++i)
            if (!fits(w[8 * g + i])) return false;
        return true;
    }
    for (int i = 0; i < 8; ++i)
        if (!fits(group_word(w, n, g, i))) return false;
    return true;
}

// Header and layout checks shared by validation and decode.
df11_status check_header(const uint8_t *c, size_t bytes, Nf12Layout &L) {
    if (!c) return report_error(DF11_E_ARG, "NF12 container pointer is NULL");
    if (bytes < kNf12Header) return report_error(DF11_E_FORMAT, "%zu bytes is shorter than the NF12 header", bytes);
    if (memcmp(c, "NF12HIPC", 8) != 0) return report_error(DF11_E_FORMAT, "bad NF12 magic");
    if (rd32(c + 8) != kNf12Version) return report_error(DF11_E_UNSUPPORTED, "NF12 version %u", rd32(c + 8));
    if (rd32(c + 12) != 0) return report_error(DF11_E_UNSUPPORTED, "NF12 flags %#x", rd32(c + 12));
    const uint64_t n = rd64(c + 16), escaped = rd64(c + 32);
    if (n > (uint64_t(1) << 46)) return report_error(DF11_E_UNSUPPORTED, "n_elems %llu", (unsigned long long)n);
    if (escaped > (n + 7) / 8) return report_error(DF11_E_FORMAT, "more outlier groups than groups");
    L = nf12_layout(n, escaped);
    if (rd64(c + 24) != L.n_groups || rd64(c + 40) != L.off_slots || rd64(c + 48) != L.off_flags ||
        rd64(c + 56) != L.off_prefix || rd64(c + 64) != L.off_escape || rd64(c + 72) != L.total)
        return report_error(DF11_E_FORMAT, "NF12 section offsets do not match the layout");
    for (uint32_t i = 80; i < kNf12Header; ++i)
        if (c[i]) return report_error(DF11_E_FORMAT, "reserved NF12 header bytes");
    return DF11_OK;
}

}  // namespace

extern "C" uint64_t df11_nf12_bound(uint64_t n) { return nf12_layout(n, (n + 7) / 8).total; }

extern "C" df11_status df11_nf12_encode(const uint16_t *words, uint64_t n, void *out_v, uint64_t out_cap,
                                        uint64_t *out_bytes, int threads) {
    if ((!words && n) || !out_v || !out_bytes) return report_error(DF11_E_ARG, "nf12_encode arguments");
    if (n > (uint64_t(1) << 46)) return report_error(DF11_E_ARG, "n_elems too large");
    if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
    uint8_t *out = (uint8_t *)out_v;
    const uint64_t G = (n + 7) / 8, n_words = (G + 63) / 64;
    std::vector<uint64_t> flags(n_words, 0);
    std::vector<uint32_t> counts(n_words, 0);
    parallel_for(n_words, threads, [&](uint64_t wd) {
        uint64_t f = 0;
        const uint64_t g_end = std::min<uint64_t>(G, 64 * wd + 64);
        for (uint64_t g = 64 * wd; g < g_end; ++g)
            if (!group_fits(words, n, g)) f |= uint64_t(1) << (g - 64 * wd);
        flags[wd] = f;
        counts[wd] = (uint32_t)__builtin_popcountll(f);
    });
    std::vector<uint64_t> before(n_words + 1, 0);
    for (uint64_t wd = 0; wd < n_words; ++wd) before[wd + 1] = before[wd] + counts[wd];
    const Nf12Layout L = nf12_layout(n, before[n_words]);
    if (out_cap < L.total) return report_error(DF11_E_ARG, "output holds %llu bytes, needs %llu",
                                               (unsigned long long)out_cap, (unsigned long long)L.total);
    memset(out, 0, kNf12Header);
    memcpy(out, "NF12HIPC", 8);
    wr32(out + 8, kNf12Version);
    wr64(out + 16, L.n);
    wr64(out + 24, L.n_groups);
    wr64(out + 32, L.n_escaped);
    wr64(out + 40, L.off_slots);
    wr64(out + 48, L.off_flags);
    wr64(out + 56, L.off_prefix);
    wr64(out + 64, L.off_escape);
    wr64(out + 72, L.total);
    // padding between and after the sections
    memset(out + L.off_slots + 12 * G, 0, L.off_flags - (L.off_slots + 12 * G));
    memset(out + L.off_flags + 8 * n_words, 0, L.off_prefix - (L.off_flags + 8 * n_words));
    memset(out + L.off_prefix + 4 * n_words, 0, L.off_escape - (L.off_prefix + 4 * n_words));
    memset(out + L.off_escape + 16 * L.n_escaped, 0, L.total - (L.off_escape + 16 * L.n_escaped));
    parallel_for(n_words, threads, [&](uint64_t wd) {
        wr64(out + L.off_flags + 8 * wd, flags[wd]);
        wr32(out + L.off_prefix + 4 * wd, (uint32_t)before[wd]);
        uint64_t e = before[wd];
        const uint64_t g_end = std::min<uint64_t>(G, 64 * wd + 64);
        for (uint64_t g = 64 * wd; g < g_end; ++g) {
            uint8_t *slot = out + L.off_slots + 12 * g;
            if ((flags[wd] >> (g - 64 * wd)) & 1u) {
                memset(slot, 0, 12);
                uint8_t *esc = out + L.off_escape + 16 * e++;
                for (int i = 0; i < 8; ++i) {
                    const uint16_t v = group_word(words, n, g, i);
                    esc[2 * i] = (uint8_t)v;
                    esc[2 * i + 1] = (uint8_t)(v >> 8);
                }
                continue;
            }
            // 8 codes of 12 bits, code i at bits 12i .. 12i+11
            uint64_t lo = 0, hi = 0;   // bits 0..63 and 64..95
            for (int i = 0; i < 8; ++i) {
                const uint16_t v = group_word(words, n, g, i);
                const uint64_t code = ((uint64_t)(v >> 15) << 11) | (v & 0x7FFu);
                const int at = 12 * i;
                if (at + 12 <= 64) {
                    lo |= code << at;
                } else if (at >= 64) {
                    hi |= code << (at - 64);
                } else {
                    lo |= code << at;
                    hi |= code >> (64 - at);
                }
            }
            memcpy(slot, &lo, 8);
            const uint32_t h32 = (uint32_t)hi;
            memcpy(slot + 8, &h32, 4);
        }
    });
    *out_bytes = L.total;
    return DF11_OK;
}

extern "C" df11_status df11_nf12_validate(const void *container, size_t bytes, uint64_t *n_elems) {
    const uint8_t *c = (const uint8_t *)container;
    Nf12Layout L;
    df11_status st = check_header(c, bytes, L);
    if (st) return st;
    if (n_elems) *n_elems = L.n;
    if (bytes < L.total) return DF11_OK;   // a header-only check
    uint64_t e = 0;
    for (uint64_t wd = 0; wd < L.n_words; ++wd) {
        if (rd32(c + L.off_prefix + 4 * wd) != e) return report_error(DF11_E_FORMAT, "NF12 prefix count of word %llu", (unsigned long long)wd);
        const uint64_t f = rd64(c + L.off_flags + 8 * wd);
        const uint64_t in_word = std::min<uint64_t>(64, L.n_groups - 64 * wd);
        if (in_word < 64 && (f >> in_word)) return report_error(DF11_E_FORMAT, "NF12 flags past the last group");
        for (uint64_t b = 0; b < in_word; ++b)
            if ((f >> b) & 1u)
                for (int k = 0; k < 12; ++k)
                    if (c[L.off_slots + 12 * (64 * wd + b) + k]) return report_error(DF11_E_FORMAT, "NF12 outlier slot not zero");
        e += (uint64_t)__builtin_popcountll(f);
    }
    if (e != L.n_escaped) return report_error(DF11_E_FORMAT, "NF12 flags count %llu outliers, header %llu",
                                              (unsigned long long)e, (unsigned long long)L.n_escaped);
    auto zero = [&](uint64_t a, uint64_t b) {
        for (uint64_t i = a; i < b; ++i) if (c[i]) return false;
        return true;
    };
    if (!zero(L.off_slots + 12 * L.n_groups, L.off_flags) || !zero(L.off_flags + 8 * L.n_words, L.off_prefix) ||
        !zero(L.off_prefix + 4 * L.n_words, L.off_escape) || !zero(L.off_escape + 16 * L.n_escaped, L.total))
        return report_error(DF11_E_FORMAT, "NF12 padding not zero");
    return DF11_OK;
}

extern "C" df11_status df11_nf12_decode_batch(const void *const *host_headers, const void *const *d_containers,
                                              void *const *d_outs, int n_tensors, int hip_device,
                                              hipStream_t stream) {
    if (n_tensors < 0 || (n_tensors > 0 && (!host_headers || !d_containers || !d_outs)))
        return report_error(DF11_E_ARG, "nf12_decode_batch arguments");
    std::vector<Nf12Layout> lay(n_tensors);
    for (int t = 0; t < n_tensors; ++t) {
        df11_status st = check_header((const uint8_t *)host_headers[t], kNf12Header, lay[t]);
        if (st) return st;
        if (lay[t].n == 0) continue;
        if (!d_containers[t] || !d_outs[t]) return report_error(DF11_E_ARG, "tensor %d: NULL device pointer", t);
        const uintptr_t c0 = (uintptr_t)d_containers[t], o0 = (uintptr_t)d_outs[t];
        if ((c0 & 15) || (o0 & 15)) return report_error(DF11_E_ARG, "tensor %d: device pointers must be 16-byte aligned", t);
        if (c0 < o0 + 2 * lay[t].n && o0 < c0 + lay[t].total)
            return report_error(DF11_E_ARG, "tensor %d: output overlaps the container", t);
    }
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != hip_device && hipSetDevice(hip_device) != hipSuccess)
        return report_error(DF11_E_HIP, "hipSetDevice(%d) failed", hip_device);
    int n_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, hip_device);
    Nf12Args a;
    memset(&a, 0, sizeof a);
    auto flush = [&]() {
        if (a.n_tensors && e == hipSuccess) e = launch_nf12_decode(a, std::max(n_cu, 1) * 32, stream);
        memset(&a, 0, sizeof a);
    };
    for (int t = 0; t < n_tensors && e == hipSuccess; ++t) {
        const Nf12Layout &L = lay[t];
        if (L.n == 0) continue;
        if (a.n_tensors == (uint32_t)kNf12MaxBatch) flush();
        const uint8_t *c = (const uint8_t *)d_containers[t];
        Nf12Tensor &T = a.t[a.n_tensors++];
        T.slots = c + L.off_slots;
        T.flags = (const uint64_t *)(c + L.off_flags);
        T.prefix = (const uint32_t *)(c + L.off_prefix);
        T.escape = c + L.off_escape;
        T.out = (uint16_t *)d_outs[t];
        T.n = L.n;
        T.n_groups = L.n_groups;
        T.n_escaped = L.n_escaped;
        T.word_base = a.n_words;
        a.n_words += L.n_words;
    }
    flush();
    if (prev >= 0 && prev != hip_device) (void)hipSetDevice(prev);
    if (e != hipSuccess) return report_error(DF11_E_HIP, "NF12 decode launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

extern "C" df11_status df11_nf12_decode(const void *host_header, const void *d_container, void *d_out,
                                        int hip_device, hipStream_t stream) {
    return df11_nf12_decode_batch(&host_header, &d_container, &d_out, 1, hip_device, stream);
}
