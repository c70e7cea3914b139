// libdf11 host side: container validation, decode-table construction, plans
// and kernel launches.  The C ABI is declared in include/df11.h.
//
// Method: mlx-dfloat project page, introduction and 16-bit weight diagram
// (exponent byte coded with a variable-length prefix code, sign + fraction
// kept as a raw byte, output identical bit for bit); df11pack project page,
// "Beyond the official format" (--luts=correct: decode-table entries that no
// valid stream reaches are zero) and "Use" (verify checks structure without
// the source).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <thread>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "df11_internal.hpp"

using namespace df11;

// ------------------------------------------------------------ error text --

// (a fixed buffer: reporting an error allocates nothing)
static thread_local char g_error[640] = "no error";

df11_status df11::report_error(df11_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    snprintf(g_error, sizeof g_error, "%s: %s", df11_status_str(st), buf);
    return st;
}

template <class... A>
static df11_status fail(df11_status st, const char *fmt, A... args) {
    return report_error(st, fmt, args...);
}

#define HIP_TRY(expr)                                                              \
    do {                                                                           \
        hipError_t e_ = (expr);                                                    \
        if (e_ != hipSuccess)                                                      \
            return fail(DF11_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

extern "C" const char *df11_status_str(df11_status s) {
    switch (s) {
        case DF11_OK: return "DF11_OK";
        case DF11_E_ARG: return "DF11_E_ARG";
        case DF11_E_FORMAT: return "DF11_E_FORMAT";
        case DF11_E_UNSUPPORTED: return "DF11_E_UNSUPPORTED";
        case DF11_E_HIP: return "DF11_E_HIP";
        case DF11_E_CORRUPT: return "DF11_E_CORRUPT";
        case DF11_E_NOMEM: return "DF11_E_NOMEM";
    }
    return "DF11_E_UNKNOWN";
}

extern "C" const char *df11_last_error(void) { return g_error; }
extern "C" int df11_abi_version(void) { return DF11_ABI_VERSION; }

// ------------------------------------------------------------ the layout --

static inline uint16_t rd16(const uint8_t *p) { uint16_t v; memcpy(&v, p, 2); return v; }
static inline uint32_t rd32(const uint8_t *p) { uint32_t v; memcpy(&v, p, 4); return v; }
static inline uint64_t rd64(const uint8_t *p) { uint64_t v; memcpy(&v, p, 8); return v; }
static inline uint64_t up256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
static inline uint64_t up16(uint64_t x) { return (x + 15) & ~uint64_t(15); }

namespace {

struct Layout {
    uint64_t n, n_chunks, total_bits;
    uint64_t off_ci, off_win, off_stream, stream_bytes, off_raw, raw_bytes, total;
};

Layout layout_for(uint64_t n, uint64_t total_bits) {
    Layout L;
    L.n = n;
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

struct Meta {
    Layout L;
    uint32_t ndim;
    uint64_t dims[8];
    uint8_t code_len[256];
    uint32_t flags;
    uint8_t sha256[32];
};

// Canonical code tables from a length vector (deflate construction).
struct Canon {
    uint32_t count[kMaxLen + 2] = {};
    uint32_t first[kMaxLen + 2] = {};
    uint32_t offset[kMaxLen + 2] = {};
    uint8_t sorted[256] = {};
    int n_sym = 0;
};

Canon canonical(const uint8_t *len) {
    Canon C;
    for (int l = 1; l <= kMaxLen; ++l)
        for (int s = 0; s < 256; ++s)
            if (len[s] == l) C.sorted[C.n_sym++] = (uint8_t)s;
    for (int s = 0; s < 256; ++s)
        if (len[s]) C.count[len[s]]++;
    uint32_t code = 0, idx = 0;
    for (int l = 1; l <= kMaxLen; ++l) {
        code = (l == 1) ? 0 : (code + C.count[l - 1]) << 1;
        C.first[l] = code;
        C.offset[l] = idx;
        idx += C.count[l];
    }
    return C;
}

// Symbol of the code of length exactly l whose value is `code`, or -1.
inline int lookup(const Canon &C, int l, uint32_t code) {
    if (!C.count[l] || code < C.first[l] || code - C.first[l] >= C.count[l]) return -1;
    return C.sorted[C.offset[l] + code - C.first[l]];
}

// Validate a metadata prefix held in host memory.
df11_status parse_and_validate(const uint8_t *c, size_t bytes, Meta &M) {
    if (!c) return fail(DF11_E_ARG, "container pointer is NULL");
    if (bytes < kHeader) return fail(DF11_E_FORMAT, "%zu bytes is shorter than the header", bytes);
    if (memcmp(c, "DF11HIPC", 8) != 0) return fail(DF11_E_FORMAT, "bad magic");
    if (rd32(c + 8) != kVersion) return fail(DF11_E_UNSUPPORTED, "container version %u", rd32(c + 8));
    M.flags = rd32(c + 12);
    if (M.flags & ~DF11_FLAG_SHA256) return fail(DF11_E_UNSUPPORTED, "flags %#x", M.flags);
    if (rd32(c + 28) != kChunk) return fail(DF11_E_UNSUPPORTED, "chunk_elems %u", rd32(c + 28));
    if (c[96] != kMaxLen) return fail(DF11_E_UNSUPPORTED, "max_code_len %u", c[96]);
    if (rd16(c + 98) != kWindows) return fail(DF11_E_UNSUPPORTED, "windows %u", rd16(c + 98));
    const uint64_t n = rd64(c + 16), total_bits = rd64(c + 104);
    if (n > (uint64_t(1) << 46)) return fail(DF11_E_UNSUPPORTED, "n_elems %llu", (unsigned long long)n);
    if (total_bits > n * kMaxLen || total_bits < n)
        return fail(DF11_E_FORMAT, "total_bits %llu for %llu elements",
                    (unsigned long long)total_bits, (unsigned long long)n);
    M.L = layout_for(n, total_bits);
    const Layout &L = M.L;
    if (L.n_chunks > (1u << 24)) return fail(DF11_E_UNSUPPORTED, "%llu chunks", (unsigned long long)L.n_chunks);
    if (rd32(c + 100) != L.n_chunks) return fail(DF11_E_FORMAT, "n_chunks field");
    if (rd64(c + 112) != L.off_ci || rd64(c + 120) != L.off_win || rd64(c + 128) != 0 ||
        rd64(c + 136) != L.off_stream || rd64(c + 144) != L.stream_bytes ||
        rd64(c + 152) != L.off_raw || rd64(c + 160) != L.raw_bytes || rd64(c + 168) != L.total)
        return fail(DF11_E_FORMAT, "section offsets or sizes do not match the layout");
    M.ndim = rd32(c + 24);
    if (M.ndim > 8) return fail(DF11_E_FORMAT, "ndim %u", M.ndim);
    uint64_t prod = 1;
    for (uint32_t i = 0; i < 8; ++i) {
        M.dims[i] = rd64(c + 32 + 8 * i);
        if (i < M.ndim) prod *= M.dims[i];
        else if (M.dims[i]) return fail(DF11_E_FORMAT, "nonzero unused dim");
    }
    if ((M.ndim && prod != n) || (!M.ndim && n != 1)) return fail(DF11_E_FORMAT, "shape does not match n_elems");
    if (c[97]) return fail(DF11_E_FORMAT, "reserved header bytes");
    memcpy(M.sha256, c + 176, 32);
    if (!(M.flags & DF11_FLAG_SHA256))
        for (int i = 176; i < 208; ++i) if (c[i]) return fail(DF11_E_FORMAT, "hash bytes without the hash flag");
    for (int i = 464; i < (int)kHeader; ++i) if (c[i]) return fail(DF11_E_FORMAT, "reserved header bytes");

    memcpy(M.code_len, c + 208, 256);
    uint64_t kraft = 0, present = 0;
    for (int s = 0; s < 256; ++s) {
        if (M.code_len[s] > kMaxLen) return fail(DF11_E_FORMAT, "code length %u > 24", M.code_len[s]);
        if (M.code_len[s]) { kraft += uint64_t(1) << (kMaxLen - M.code_len[s]); ++present; }
    }
    if (n == 0 && present) return fail(DF11_E_FORMAT, "codes for an empty tensor");
    if (n && !present) return fail(DF11_E_FORMAT, "no codes");
    if (present == 1 && kraft != (uint64_t(1) << (kMaxLen - 1)))
        return fail(DF11_E_FORMAT, "single symbol must have a 1-bit code");
    if (present >= 2 && kraft != (uint64_t(1) << kMaxLen))
        return fail(DF11_E_FORMAT, "Kraft sum is not 1");

    if (bytes < L.off_stream) return fail(DF11_E_FORMAT, "prefix of %zu bytes does not hold the index (%llu)",
                                          bytes, (unsigned long long)L.off_stream);
    // chunk index and windows
    for (uint64_t ch = 0; ch <= L.n_chunks; ++ch) {
        const uint8_t *e = c + L.off_ci + ch * 16;
        const uint64_t sb = rd64(e), oe = rd64(e + 8);
        if (ch == L.n_chunks) {
            if (sb != total_bits || oe != n) return fail(DF11_E_FORMAT, "bad sentinel");
            break;
        }
        if (oe != ch * kChunk) return fail(DF11_E_FORMAT, "chunk %llu out_elem", (unsigned long long)ch);
        const uint64_t b1 = rd64(e + 16);
        const uint64_t elems = std::min<uint64_t>(kChunk, n - ch * kChunk);
        if (sb > b1 || b1 - sb < elems || b1 - sb > elems * kMaxLen)
            return fail(DF11_E_FORMAT, "chunk %llu bit range", (unsigned long long)ch);
        const uint32_t nbits = (uint32_t)(b1 - sb);   // <= 24 * kChunk, checked above
        uint64_t sum = 0;
        for (int i = 0; i < kWindows; ++i) {
            const unsigned ent = rd16(c + L.off_win + (ch * kWindows + i) * 2);
            const unsigned cnt = ent & kWinCntMask, gap = ent >> kWinGapShift;
            sum += cnt;
            const uint64_t ws = sb + window_edge(nbits, i), we = sb + window_edge(nbits, i + 1);
            if (cnt == 0) {
                if (gap != 0) return fail(DF11_E_FORMAT, "chunk %llu window %d: gap without codes", (unsigned long long)ch, i);
                continue;
            }
            if (gap >= (unsigned)kMaxLen || ws >= b1 || ws + gap >= we || cnt > we - ws - gap)
                return fail(DF11_E_FORMAT, "chunk %llu window %d: gap %u cnt %u", (unsigned long long)ch, i, gap, cnt);
        }
        if (sum != elems) return fail(DF11_E_FORMAT, "chunk %llu: window counts sum to %llu, not %llu",
                                      (unsigned long long)ch, (unsigned long long)sum, (unsigned long long)elems);
    }
    // padding of the stream and the raw section, when the bytes are there
    if (bytes >= L.total) {
        for (uint64_t b = total_bits; b < (total_bits + 7) / 8 * 8; ++b)
            if ((c[L.off_stream + b / 8] >> (7 - b % 8)) & 1) return fail(DF11_E_FORMAT, "stream padding");
        for (uint64_t i = (total_bits + 7) / 8; i < L.stream_bytes; ++i)
            if (c[L.off_stream + i]) return fail(DF11_E_FORMAT, "stream padding");
        for (uint64_t i = n; i < L.raw_bytes; ++i)
            if (c[L.off_raw + i]) return fail(DF11_E_FORMAT, "raw padding");
    }
    return DF11_OK;
}

void fill_info(const Meta &M, df11_tensor_info *info) {
    memset(info, 0, sizeof *info);
    const Layout &L = M.L;
    info->n_elems = L.n;
    info->ndim = M.ndim;
    info->n_chunks = (uint32_t)L.n_chunks;
    memcpy(info->dims, M.dims, sizeof M.dims);
    info->total_bits = L.total_bits;
    info->container_bytes = L.total;
    info->meta_bytes = L.off_stream;
    // what a decode reads: the plan's 64-byte record per chunk (the kernel
    // never reads the container's chunk index), one 16-bit entry per window,
    // the code bits and one raw byte per element
    info->bytes_read_per_decode =
        L.n_chunks * sizeof(ChunkRec) + L.n_chunks * kWindows * 2 + (L.total_bits + 7) / 8 + L.n;
    memcpy(info->code_len, M.code_len, 256);
    info->flags = M.flags;
    memcpy(info->sha256, M.sha256, 32);
}

}  // namespace

void df11::build_lut(const uint8_t *len, LutRecord &R) {
    memset(&R, 0, sizeof R);
    Canon C = canonical(len);
    for (int i = 0; i < C.n_sym; ++i) R.sorted[i] = rot_exp(C.sorted[i]);
    for (int s = 0; s < 256; ++s) R.len[rot_exp(s)] = len[s];
    for (int l = 0; l < 32; ++l) { R.lim[l] = 0xFFFFFFFFu; R.base[l] = 0; }
    R.lim[0] = 0;
    for (int l = 1; l <= kMaxLen; ++l) {
        R.lim[l] = (C.first[l] + C.count[l]) << (kMaxLen - l);
        R.base[l] = (int32_t)C.offset[l] - (int32_t)C.first[l];
    }
    // First level: greedily resolve up to three whole codes inside the next
    // kL1Bits bits.  A prefix that starts with no code of <= kL1Bits bits
    // (or that no valid stream holds) gets a subtable entry below.
    for (uint32_t v = 0; v < (uint32_t)kL1Size; ++v) {
        int pos = 0, n = 0;
        uint32_t syms = 0;
        while (n < kMaxPerLookup) {
            int found = -1, flen = 0;
            for (int l = 1; l <= kL1Bits - pos && found < 0; ++l) {
                uint32_t code = (v >> (kL1Bits - pos - l)) & ((1u << l) - 1);
                found = lookup(C, l, code);
                flen = l;
            }
            if (found < 0) break;
            syms |= (uint32_t)rot_exp((unsigned)found) << (8 * n);
            pos += flen;
            ++n;
        }
        // indexed by the 10 bits in stream order, first bit lowest (the
        // decoder reads its code words least significant bit first)
        const uint32_t rv = __builtin_bitreverse32(v) >> (32 - kL1Bits);
        R.l1[rv] = n ? (syms | ((uint32_t)pos << kEntLenShift) | ((uint32_t)n << kEntCountShift)) : 0u;
    }
    // Second level: a subtable per prefix whose first code is longer than
    // kL1Bits (layout in df11_internal.hpp), in canonical order, so that the
    // shorter and more frequent long codes get a subtable first.
    uint32_t used = 2;
    for (uint32_t v = 0; v < (uint32_t)kL1Size; ++v) {
        const uint32_t rv = __builtin_bitreverse32(v) >> (32 - kL1Bits);
        if (R.l1[rv]) continue;
        uint32_t maxlen = 0;
        for (int l = kL1Bits + 1; l <= kMaxLen; ++l) {
            const uint64_t lo = (uint64_t)v << (l - kL1Bits), hi = (uint64_t)(v + 1) << (l - kL1Bits);
            if (C.count[l] && lo < (uint64_t)C.first[l] + C.count[l] && hi > C.first[l]) maxlen = (uint32_t)l;
        }
        const uint32_t k = maxlen ? std::min<uint32_t>(maxlen, kL2Bits) - kL1Bits : 1u;
        uint32_t off = 0;
        if (maxlen && used + (1u << k) <= (uint32_t)kL2Max) {
            off = used;
            used += 1u << k;
            for (uint32_t j = 0; j < (1u << k); ++j) {
                // j's bits in stream order, first bit lowest
                for (uint32_t l = kL1Bits + 1; l <= kL1Bits + k; ++l) {
                    const uint32_t ext = l - kL1Bits;
                    const uint32_t tail = __builtin_bitreverse32(j & ((1u << ext) - 1u)) >> (32 - ext);
                    const int s = lookup(C, (int)l, (v << ext) | tail);
                    if (s >= 0) {
                        R.l2[off + j] = (uint16_t)(rot_exp((unsigned)s) | ((l | 32u) << 8));
                        break;
                    }
                }
            }
        }
        const uint32_t last_bit = (rv >> (kL1Bits - 1)) & 1u;
        const uint32_t F = 2u + 2u * off - last_bit;
        R.l1[rv] = (F << 16) | (k + 1u);
    }
}

extern "C" df11_status df11_validate(const void *host_meta, size_t bytes, df11_tensor_info *info) {
    Meta M;
    df11_status st = parse_and_validate((const uint8_t *)host_meta, bytes, M);
    if (st) return st;
    if (info) fill_info(M, info);
    return DF11_OK;
}

extern "C" df11_status df11_verify_words(const void *host_meta, size_t bytes, const uint16_t *host_words,
                                         uint64_t n) {
    Meta M;
    df11_status st = parse_and_validate((const uint8_t *)host_meta, bytes, M);
    if (st) return st;
    if (!(M.flags & DF11_FLAG_SHA256)) return fail(DF11_E_UNSUPPORTED, "the container holds no source hash");
    if (n != M.L.n || (!host_words && n))
        return fail(DF11_E_ARG, "%llu words for a container of %llu", (unsigned long long)n,
                    (unsigned long long)M.L.n);
    uint8_t h[32];
    sha256(host_words, 2 * n, h);   // the words' bytes, low byte first (little-endian host)
    if (memcmp(h, M.sha256, 32) != 0) return fail(DF11_E_CORRUPT, "the words' SHA-256 differs from the header's");
    return DF11_OK;
}

extern "C" uint64_t df11_container_bound(uint64_t n) {
    return layout_for(n, n * kMaxLen).total;
}

// ------------------------------------------------------------------ plans --

struct df11_plan_s {
    int device = 0;
    int n_tensors = 0;
    int n_cu = 0;
    std::vector<Meta> meta;
    std::vector<uint64_t> first_rec;   // per tensor (and one past the last): first chunk record
    void *d_block = nullptr;
    ChunkRec *d_recs = nullptr;
    LutRecord *d_luts = nullptr;
    uint32_t *d_status = nullptr;
    uint32_t *d_work = nullptr;              // kWorkSlots ticket counters
    uint32_t *h_fin = nullptr;               // kWorkSlots completion words (pinned host memory)
    uint32_t *d_fin = nullptr;               // the same words, as the device addresses them
    int wgs_cap = 0;                         // decode workgroups per CU (0: as many as fit)
    std::mutex slot_mu;
    SlotTable slots;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) err = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// A ticket counter no running launch of the plan holds, for a launch on
// `stream` (fills a.work, a.fin, a.launch_id).  Waits on the host while every
// slot is held (kWorkSlots launches of the plan queued and not finished),
// for at most a minute.
df11_status take_work_slot(df11_plan_s *p, hipStream_t stream, DecodeArgs &a, int &slot) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
    const bool capture = cs != hipStreamCaptureStatusNone;
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
        {
            std::lock_guard<std::mutex> lock(p->slot_mu);
            uint32_t id = 0;
            slot = p->slots.acquire(p->h_fin, capture, &id);
            if (slot >= 0) {
                a.work = p->d_work + kWorkStride * (uint32_t)slot;
                a.fin = p->d_fin + slot;
                a.launch_id = id;
                return DF11_OK;
            }
            if (capture && p->slots.n_graph >= kGraphSlotsMax)
                return fail(DF11_E_UNSUPPORTED, "%u captured decodes already hold counters of this plan", kGraphSlotsMax);
        }
        if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60))
            return fail(DF11_E_HIP, "no ticket counter came free in 60 s: %u decodes of this plan queued and unfinished",
                        kWorkSlots);
        std::this_thread::sleep_for(std::chrono::microseconds(20));
    }
}

void give_back_slot(df11_plan_s *p, int slot) {
    std::lock_guard<std::mutex> lock(p->slot_mu);
    p->slots.release(slot);
}

int grid_for(const df11_plan_s *p, uint64_t items) {
    uint64_t per_cu = (uint64_t)decode_wgs_per_cu();
    if (p->wgs_cap > 0) per_cu = std::min<uint64_t>(per_cu, (uint64_t)p->wgs_cap);
    const uint64_t resident = (uint64_t)p->n_cu * per_cu;
    return (int)std::max<uint64_t>(1, std::min<uint64_t>(items, resident));
}

}  // namespace

extern "C" df11_status df11_plan(const void *const *host_meta, const size_t *host_meta_bytes,
                                 int n_tensors, int hip_device, uint32_t flags, df11_plan_t *out) {
    if (!out) return fail(DF11_E_ARG, "out is NULL");
    *out = nullptr;
    if (n_tensors <= 0 || !host_meta || !host_meta_bytes)
        return fail(DF11_E_ARG, "need at least one tensor");
    if (flags != 0) return fail(DF11_E_ARG, "flags must be 0");
    df11_plan_s *p = new (std::nothrow) df11_plan_s;
    if (!p) return fail(DF11_E_NOMEM, "plan");
    p->device = hip_device;
    p->n_tensors = n_tensors;
    p->meta.resize(n_tensors);
    for (int t = 0; t < n_tensors; ++t) {
        df11_status st = parse_and_validate((const uint8_t *)host_meta[t], host_meta_bytes[t], p->meta[t]);
        if (st) {
            const size_t used = strlen(g_error);
            snprintf(g_error + used, sizeof g_error - used, " (tensor %d)", t);
            delete p;
            return st;
        }
    }
    // host images of the decode tables and the chunk records (plan order)
    std::vector<LutRecord> luts(n_tensors);
    std::vector<ChunkRec> recs;
    p->first_rec.push_back(0);
    for (int t = 0; t < n_tensors; ++t) {
        const Layout &L = p->meta[t].L;
        build_lut(p->meta[t].code_len, luts[t]);
        const uint8_t *ci = (const uint8_t *)host_meta[t] + L.off_ci;
        for (uint64_t ch = 0; ch < L.n_chunks; ++ch) {
            const uint64_t b0 = rd64(ci + 16 * ch), b1 = rd64(ci + 16 * (ch + 1));
            const uint64_t elem0 = ch * kChunk;
            const uint64_t sb = L.stream_bytes;
            // staged bytes: the chunk's stream bytes plus 127 bits of slack,
            // rounded out to 16 bytes, inside the stream section
            const uint64_t s0 = std::min<uint64_t>((b0 >> 3) & ~uint64_t(15), sb - 16);
            const uint64_t s_end = std::max<uint64_t>(std::min<uint64_t>((((b1 + 127) >> 3) + 15) & ~uint64_t(15), sb), s0 + 16);
            ChunkRec r;
            memset(&r, 0, sizeof r);
            r.stream_off = L.off_stream + s0;
            r.raw_off = L.off_raw + elem0;
            r.win_off = L.off_win + ch * kWindows * 2;
            r.rel0 = (uint32_t)(b0 - 8 * s0);
            r.nbits = (uint32_t)(b1 - b0);
            r.s_len = (uint32_t)std::min<uint64_t>(s_end - s0, kCodeCap) | (s_end <= s0 + kCodeCap ? kStagedBit : 0u);
            r.nc = (uint32_t)std::min<uint64_t>(kChunk, L.n - elem0);
            r.raw_left = (uint32_t)std::min<uint64_t>(L.raw_bytes - elem0, 2 * kChunk);
            r.n_words = (uint32_t)std::min<uint64_t>((sb - s0) / 4, uint64_t(1) << 25);
            r.tensor = (uint32_t)t;
            r.chunk = (uint32_t)ch;
            recs.push_back(r);
        }
        p->first_rec.push_back(recs.size());
    }

    const size_t off_recs = 0;
    const size_t off_luts = up256(off_recs + sizeof(ChunkRec) * std::max<size_t>(1, recs.size()));
    const size_t off_status = up256(off_luts + sizeof(LutRecord) * n_tensors);
    const size_t off_work = off_status + 256;
    const size_t total = off_work + sizeof(uint32_t) * kWorkStride * kWorkSlots;
    std::vector<uint8_t> image(total, 0);
    if (!recs.empty()) memcpy(image.data() + off_recs, recs.data(), sizeof(ChunkRec) * recs.size());
    memcpy(image.data() + off_luts, luts.data(), sizeof(LutRecord) * n_tensors);

    DeviceGuard guard(hip_device);
    if (guard.err != hipSuccess) { delete p; return fail(DF11_E_HIP, "hipSetDevice(%d): %s", hip_device, hipGetErrorString(guard.err)); }
    int n_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, hip_device);
    if (e != hipSuccess || n_cu <= 0) { delete p; return fail(DF11_E_HIP, "device %d: no compute units (%s)", hip_device, hipGetErrorString(e)); }
    p->n_cu = n_cu;
    e = hipMalloc(&p->d_block, total);
    if (e != hipSuccess) { delete p; return fail(DF11_E_HIP, "hipMalloc(%zu): %s", total, hipGetErrorString(e)); }
    e = hipMemcpy(p->d_block, image.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(p->d_block);
        delete p;
        return fail(DF11_E_HIP, "hipMemcpy: %s", hipGetErrorString(e));
    }
    uint8_t *base = (uint8_t *)p->d_block;
    p->d_recs = (ChunkRec *)(base + off_recs);
    p->d_luts = (LutRecord *)(base + off_luts);
    p->d_status = (uint32_t *)(base + off_status);
    p->d_work = (uint32_t *)(base + off_work);
    // the slots' completion words: coherent pinned host memory the decode
    // kernel writes at the end of each launch
    e = hipHostMalloc((void **)&p->h_fin, sizeof(uint32_t) * kWorkSlots, hipHostMallocCoherent | hipHostMallocMapped);
    if (e == hipSuccess) {
        memset(p->h_fin, 0, sizeof(uint32_t) * kWorkSlots);
        e = hipHostGetDevicePointer((void **)&p->d_fin, p->h_fin, 0);
    }
    if (e != hipSuccess) {
        df11_plan_destroy(p);
        return fail(DF11_E_HIP, "completion words: %s", hipGetErrorString(e));
    }
    *out = p;
    return DF11_OK;
}

extern "C" void df11_plan_destroy(df11_plan_t p) {
    if (!p) return;
    DeviceGuard guard(p->device);
    if (p->d_block) (void)hipFree(p->d_block);
    if (p->h_fin) (void)hipHostFree(p->h_fin);
    delete p;
}

extern "C" df11_status df11_plan_info(df11_plan_t p, int tensor, df11_tensor_info *info) {
    if (!p || !info || tensor < 0 || tensor >= p->n_tensors) return fail(DF11_E_ARG, "plan_info arguments");
    fill_info(p->meta[tensor], info);
    return DF11_OK;
}

extern "C" df11_status df11_plan_set_wgs_per_cu(df11_plan_t p, int wgs_per_cu) {
    if (!p || wgs_per_cu < 0) return fail(DF11_E_ARG, "df11_plan_set_wgs_per_cu arguments");
    p->wgs_cap = wgs_per_cu;
    return DF11_OK;
}

static df11_status check_ptrs(const df11_plan_s *p, int t, const void *cont, const void *out) {
    if (p->meta[t].L.n == 0) return DF11_OK;
    if (!cont || !out) return fail(DF11_E_ARG, "tensor %d: NULL pointer", t);
    if (((uintptr_t)cont & 15) || ((uintptr_t)out & 15))
        return fail(DF11_E_ARG, "tensor %d: pointers must be 16-byte aligned", t);
    const uint64_t cb = p->meta[t].L.total, ob = p->meta[t].L.n * 2;
    const uintptr_t c0 = (uintptr_t)cont, o0 = (uintptr_t)out;
    if (c0 < o0 + ob && o0 < c0 + cb) return fail(DF11_E_ARG, "tensor %d: output overlaps the container", t);
    return DF11_OK;
}

extern "C" df11_status df11_decode(df11_plan_t p, int tensor, const void *d_container, void *d_out,
                                   hipStream_t stream) {
    if (!p || tensor < 0 || tensor >= p->n_tensors) return fail(DF11_E_ARG, "decode arguments");
    df11_status st = check_ptrs(p, tensor, d_container, d_out);
    if (st) return st;
    const uint32_t n_chunks = (uint32_t)p->meta[tensor].L.n_chunks;
    if (n_chunks == 0) return DF11_OK;
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.recs = p->d_recs + p->first_rec[tensor];
    a.luts = p->d_luts;
    a.status = p->d_status;
    a.n_items = n_chunks;
    a.tensor_base = (uint32_t)tensor;
    a.containers[0] = (const uint8_t *)d_container;
    a.outs[0] = (uint16_t *)d_out;
    DeviceGuard guard(p->device);
    if (guard.err != hipSuccess) return fail(DF11_E_HIP, "hipSetDevice: %s", hipGetErrorString(guard.err));
    int slot = -1;
    st = take_work_slot(p, stream, a, slot);
    if (st) return st;
    const hipError_t e = launch_decode(a, grid_for(p, n_chunks), stream);
    if (e != hipSuccess) {
        give_back_slot(p, slot);
        return fail(DF11_E_HIP, "decode launch: %s", hipGetErrorString(e));
    }
    return DF11_OK;
}

extern "C" df11_status df11_decode_batch(df11_plan_t p, const void *const *d_containers,
                                         void *const *d_outs, hipStream_t stream) {
    if (!p || !d_containers || !d_outs) return fail(DF11_E_ARG, "decode_batch arguments");
    for (int t = 0; t < p->n_tensors; ++t) {
        df11_status st = check_ptrs(p, t, d_containers[t], d_outs[t]);
        if (st) return st;
    }
    DeviceGuard guard(p->device);
    if (guard.err != hipSuccess) return fail(DF11_E_HIP, "hipSetDevice: %s", hipGetErrorString(guard.err));
    for (int g = 0; g * DF11_MAX_BATCH < p->n_tensors; ++g) {
        const int t_end = std::min(p->n_tensors, (g + 1) * DF11_MAX_BATCH);
        const uint64_t r0 = p->first_rec[g * DF11_MAX_BATCH], r1 = p->first_rec[t_end];
        if (r1 == r0) continue;
        DecodeArgs a;
        memset(&a, 0, sizeof a);
        a.recs = p->d_recs + r0;
        a.luts = p->d_luts;
        a.status = p->d_status;
        a.n_items = (uint32_t)(r1 - r0);
        a.tensor_base = (uint32_t)(g * DF11_MAX_BATCH);
        for (int t = (int)g * DF11_MAX_BATCH; t < t_end; ++t) {
            a.containers[t - g * DF11_MAX_BATCH] = (const uint8_t *)d_containers[t];
            a.outs[t - g * DF11_MAX_BATCH] = (uint16_t *)d_outs[t];
        }
        int slot = -1;
        df11_status st = take_work_slot(p, stream, a, slot);
        if (st) return st;
        const hipError_t e = launch_decode(a, grid_for(p, a.n_items), stream);
        if (e != hipSuccess) {
            give_back_slot(p, slot);
            return fail(DF11_E_HIP, "decode launch: %s", hipGetErrorString(e));
        }
    }
    return DF11_OK;
}

extern "C" df11_status df11_bw_control(const void *d_src, uint64_t src_bytes, void *d_dst, uint64_t dst_bytes,
                                       int hip_device, hipStream_t stream) {
    if (!d_src || !d_dst) return fail(DF11_E_ARG, "NULL buffer");
    if (((uintptr_t)d_src | (uintptr_t)d_dst) & 15) return fail(DF11_E_ARG, "buffers must be 16-byte aligned");
    if (src_bytes < 16 || dst_bytes < 16 || (src_bytes | dst_bytes) & 15)
        return fail(DF11_E_ARG, "sizes must be positive multiples of 16");
    if (src_bytes >= (uint64_t(1) << 40) || dst_bytes >= (uint64_t(1) << 40))
        return fail(DF11_E_ARG, "sizes must be below 2^40 bytes");
    // (output unit i reads source unit floor(i * src / dst): with a smaller
    // output most of the source would go unread)
    if (src_bytes > dst_bytes)
        return fail(DF11_E_ARG, "src_bytes above dst_bytes: a decode writes more than it reads");
    const uintptr_t s0 = (uintptr_t)d_src, d0 = (uintptr_t)d_dst;
    if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return fail(DF11_E_ARG, "regions overlap");
    DeviceGuard guard(hip_device);
    if (guard.err != hipSuccess) return fail(DF11_E_HIP, "hipSetDevice(%d): %s", hip_device, hipGetErrorString(guard.err));
    int n_cu = 0;
    HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, hip_device));
    if (n_cu <= 0) return fail(DF11_E_HIP, "device %d: no compute units", hip_device);
    HIP_TRY(launch_bw_control(d_src, src_bytes, d_dst, dst_bytes, n_cu * 32, stream));
    return DF11_OK;
}

extern "C" df11_status df11_check(df11_plan_t p, hipStream_t stream) {
    if (!p) return fail(DF11_E_ARG, "plan is NULL");
    DeviceGuard guard(p->device);
    if (guard.err != hipSuccess) return fail(DF11_E_HIP, "hipSetDevice: %s", hipGetErrorString(guard.err));
    HIP_TRY(hipStreamSynchronize(stream));
    uint32_t flag = 0;
    HIP_TRY(hipMemcpy(&flag, p->d_status, sizeof flag, hipMemcpyDeviceToHost));
    if (flag) {
        const uint32_t zero = 0;
        HIP_TRY(hipMemcpy(p->d_status, &zero, sizeof zero, hipMemcpyHostToDevice));
        return fail(DF11_E_CORRUPT, "a decode found a window whose codes did not end where the next window's first code starts");
    }
    return DF11_OK;
}
