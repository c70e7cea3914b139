// GPU encoder for gfx950: BF16 words in device memory -> version-4 container
// in device memory, byte for byte the container the host encoder writes.
//
// Method (mlx-dfloat project page, introduction and 16-bit weight diagram):
// each exponent byte gets a length-limited canonical prefix code, the sign +
// 7-bit fraction stay as one raw byte.  The df11pack page ("Measured")
// makes compression time the cost to cut; here the element-wise passes run
// on the GPU and only the 256-symbol code is built on the host:
//
//   1. histogram of the exponent byte (one read of the words);
//   -- the host builds the code (package-merge, canonical values), the layout
//      from the total bit count sum(f * len), and the header;
//   2. per-chunk bit counts, written where the chunk index goes;
//   3. one workgroup turns them into start bits (the chunk index);
//   4. one workgroup per chunk: every lane packs the codes of 128 consecutive
//      elements into 32-bit words of the stream (whole words with plain
//      stores, the two it may share with its neighbours with an atomic OR
//      into the zeroed section), counts the codes that start in each of the
//      chunk's 512 windows and the offset of each window's first code (in
//      LDS), and writes the elements' raw bytes.
//
// Bound by HBM traffic: the words are read three times (2 bytes each) and
// about 1.36 bytes per element are written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "df11_internal.hpp"

namespace df11 {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

constexpr int kEncThreads = 256;
constexpr int kPerLane = kChunk / kEncThreads;   // 128 elements per lane
constexpr int kHistCopies = 16;                  // LDS copies of the histogram (lane % 16 picks one)

struct CodeTable {
    uint32_t code[256];
    uint8_t len[256];
};

__device__ __forceinline__ uint32_t bswap32(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0x00010203u); }

// The 8 words of a 16-byte group, one at a time (low half first).
__device__ __forceinline__ uint32_t word_of(const u32x4 &v, int i) {
    const uint32_t d = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (i & 1) ? d >> 16 : d & 0xFFFFu;
}

// 1. exponent histogram (u32 counters per workgroup, summed into u64)
__global__ __launch_bounds__(kEncThreads) void enc_hist(const GLOBAL uint16_t *w, uint64_t n,
                                                        GLOBAL unsigned long long *hist) {
    // (each copy is one entry longer than the 256 bins, so that the copies of
    // a bin fall in different LDS banks; one copy per lane measured slower)
    __shared__ uint32_t h[kHistCopies][257];
    for (int i = threadIdx.x; i < kHistCopies * 257; i += kEncThreads) (&h[0][0])[i] = 0;
    __syncthreads();
    uint32_t *mine = h[threadIdx.x % kHistCopies];
    const uint64_t stride = (uint64_t)gridDim.x * kEncThreads * 8;
    for (uint64_t j = ((uint64_t)blockIdx.x * kEncThreads + threadIdx.x) * 8; j < n; j += stride) {
        if (j + 8 <= n) {
            const u32x4 v = *reinterpret_cast<const GLOBAL u32x4 *>(w + j);
#pragma unroll
            for (int i = 0; i < 8; ++i) atomicAdd(&mine[(word_of(v, i) >> 7) & 0xFFu], 1u);
        } else {
            for (uint64_t k = j; k < n; ++k) atomicAdd(&mine[(w[k] >> 7) & 0xFFu], 1u);
        }
    }
    __syncthreads();
    uint32_t sum = 0;
    for (int c = 0; c < kHistCopies; ++c) sum += h[(c + threadIdx.x) % kHistCopies][threadIdx.x];
    if (sum) __hip_atomic_fetch_add(&hist[threadIdx.x], (unsigned long long)sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane tid's elements of chunk c: [j0, j0 + m).
struct LaneRange {
    uint64_t j0;
    uint32_t m;
};
__device__ __forceinline__ LaneRange lane_range(uint64_t c, uint32_t tid, uint64_t n) {
    const uint64_t j0 = c * kChunk + (uint64_t)tid * kPerLane;
    return LaneRange{j0, j0 < n ? (uint32_t)min((uint64_t)kPerLane, n - j0) : 0u};
}

// Calls f(i, word) for the lane's elements in order (16-byte loads when the
// whole group of 8 is there).
template <class F>
__device__ __forceinline__ void for_each_word(const GLOBAL uint16_t *w, LaneRange r, F &&f) {
    for (uint32_t g = 0; g < r.m; g += 8) {
        if (g + 8 <= r.m) {
            const u32x4 v = *reinterpret_cast<const GLOBAL u32x4 *>(w + r.j0 + g);
#pragma unroll
            for (int i = 0; i < 8; ++i) f(g + i, word_of(v, i));
        } else {
            for (uint32_t i = g; i < r.m; ++i) f(i, (uint32_t)w[r.j0 + i]);
        }
    }
}

// Exclusive prefix sum over the workgroup's 256 lanes (LDS, both buffers of
// `s` used in turn); also returns the total.
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t (&s)[2][kEncThreads], uint32_t &total) {
    const uint32_t tid = threadIdx.x;
    s[0][tid] = v;
    __syncthreads();
    int src = 0;
    for (uint32_t d = 1; d < kEncThreads; d <<= 1) {
        const uint32_t x = s[src][tid] + (tid >= d ? s[src][tid - d] : 0u);
        s[src ^ 1][tid] = x;
        src ^= 1;
        __syncthreads();
    }
    total = s[src][kEncThreads - 1];
    return s[src][tid] - v;
}

// 2. bits of each chunk, into the chunk index's start-bit slots
__global__ __launch_bounds__(kEncThreads) void enc_chunk_bits(const GLOBAL uint16_t *w, uint64_t n, CodeTable T,
                                                              GLOBAL uint64_t *ci) {
    __shared__ uint8_t len[256];
    __shared__ uint32_t s[2][kEncThreads];
    len[threadIdx.x] = T.len[threadIdx.x];
    __syncthreads();
    // (the order does not matter for a sum: each load instruction covers 4 KiB
    // of consecutive words across the workgroup)
    uint32_t bits = 0;
    const uint64_t c0 = (uint64_t)blockIdx.x * kChunk;
    const uint64_t cend = min(n, c0 + kChunk);
    for (uint64_t j = c0 + 8 * threadIdx.x; j < cend; j += 8 * kEncThreads) {
        if (j + 8 <= cend) {
            const u32x4 v = *reinterpret_cast<const GLOBAL u32x4 *>(w + j);
#pragma unroll
            for (int i = 0; i < 8; ++i) bits += len[(word_of(v, i) >> 7) & 0xFFu];
        } else {
            for (uint64_t k = j; k < cend; ++k) bits += len[(w[k] >> 7) & 0xFFu];
        }
    }
    uint32_t total;
    block_exclusive(bits, s, total);
    if (threadIdx.x == 0) ci[2 * (uint64_t)blockIdx.x] = total;
}

// 3. start bits: exclusive prefix sum of the chunk bit counts, in place,
// with each chunk's first element and the sentinel {total bits, n}
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void enc_scan(GLOBAL uint64_t *ci, uint64_t n_chunks, uint64_t n) {
    __shared__ uint64_t s[2][kScanThreads];
    __shared__ uint64_t carry;
    const uint32_t tid = threadIdx.x;
    if (tid == 0) carry = 0;
    for (uint64_t base = 0; base < n_chunks; base += kScanThreads) {
        __syncthreads();
        const uint64_t c = base + tid;
        const uint64_t v = c < n_chunks ? ci[2 * c] : 0;
        s[0][tid] = v;
        __syncthreads();
        int src = 0;
        for (uint32_t d = 1; d < kScanThreads; d <<= 1) {
            const uint64_t x = s[src][tid] + (tid >= d ? s[src][tid - d] : 0u);
            s[src ^ 1][tid] = x;
            src ^= 1;
            __syncthreads();
        }
        if (c < n_chunks) {
            ci[2 * c] = carry + s[src][tid] - v;
            ci[2 * c + 1] = c * kChunk;
        }
        __syncthreads();
        if (tid == kScanThreads - 1) carry += s[src][tid];
    }
    __syncthreads();
    if (tid == 0) {
        ci[2 * n_chunks] = carry;
        ci[2 * n_chunks + 1] = n;
    }
}

struct PackArgs {
    const GLOBAL uint16_t *w;
    uint64_t n;
    const GLOBAL uint64_t *ci;   // the chunk index (start bits)
    GLOBAL uint32_t *stream;     // the stream section, zeroed, as 32-bit words
    GLOBAL uint32_t *win;        // the window section
    GLOBAL uint8_t *raw;         // the raw section
};

// A lane's words for its passes: held in registers when the lane has all 128
// (every lane but some of a tensor's last chunk), else read again from
// global memory on each pass.
struct LaneWords {
    u32x4 v[kPerLane / 8];
    const GLOBAL uint16_t *w;
    LaneRange r;
    bool full;
    __device__ __forceinline__ LaneWords(const GLOBAL uint16_t *w_, LaneRange r_)
        : w(w_), r(r_), full(r_.m == (uint32_t)kPerLane) {
        if (full) {
#pragma unroll
            for (int g = 0; g < kPerLane / 8; ++g) v[g] = *reinterpret_cast<const GLOBAL u32x4 *>(w + r.j0 + 8 * g);
        }
    }
    template <class F>
    __device__ __forceinline__ void each(F &&f) const {
        if (full) {
#pragma unroll
            for (int g = 0; g < kPerLane / 8; ++g) {
#pragma unroll
                for (int i = 0; i < 8; ++i) f((uint32_t)(8 * g + i), word_of(v[g], i));
            }
        } else {
            for_each_word(w, r, f);
        }
    }
};

// 4. one chunk: codes into the stream, the window index, the raw bytes
__global__ __launch_bounds__(kEncThreads) void enc_pack(PackArgs a, CodeTable T) {
    __shared__ uint32_t code[256];
    __shared__ uint8_t len[256];
    __shared__ uint32_t cnt[kWindows], gap[kWindows];
    __shared__ uint32_t s[2][kEncThreads];
    __shared__ uint8_t last_len[kEncThreads];
    const uint32_t tid = threadIdx.x;
    const uint64_t c = blockIdx.x;
    code[tid] = T.code[tid];
    len[tid] = T.len[tid];
    cnt[tid] = cnt[tid + kEncThreads] = 0;
    gap[tid] = gap[tid + kEncThreads] = 0;
    __syncthreads();

    const LaneRange r = lane_range(c, tid, a.n);
    const LaneWords words(a.w, r);
    // this lane's bits and its last element's code length, for its neighbours
    uint32_t bits = 0, lastl = 0;
    words.each([&](uint32_t, uint32_t x) {
        lastl = len[(x >> 7) & 0xFFu];
        bits += lastl;
    });
    last_len[tid] = (uint8_t)lastl;
    uint32_t nbits_scan;
    const uint32_t p0 = block_exclusive(bits, s, nbits_scan);   // (its barriers publish last_len)

    const uint64_t b0 = a.ci[2 * c];
    const uint32_t N = (uint32_t)(a.ci[2 * c + 2] - b0);   // the chunk's bits (= nbits_scan)
    if (r.m) {
        uint64_t G = b0 + p0;            // stream position of the next code
        uint64_t k = G >> 5;             // its word
        uint32_t o = (uint32_t)(G & 31); // its bit in the word, first stream bit highest
        uint32_t cur = 0;
        bool first_word = true;
        uint32_t pos = p0;                                   // chunk-relative start of the next code
        uint32_t prev_len = tid ? last_len[tid - 1] : 0u;     // the code before it
        // the window of the lane's first code: the last one that starts at or
        // before it (windows start at floor(i N / 512)); then moved forward
        uint32_t wi = min((uint32_t)kWindows - 1u, (kWindows * (p0 + 1u) - 1u) / N);
        uint32_t run_w = ~0u, run = 0;
        words.each([&](uint32_t, uint32_t x) {
            const uint32_t e = (x >> 7) & 0xFFu;
            const uint32_t L = len[e];
            while (wi + 1u < (uint32_t)kWindows && window_edge(N, wi + 1u) <= pos) ++wi;
            const uint32_t edge = window_edge(N, wi);
            if (pos == 0 || edge > pos - prev_len) gap[wi] = pos - edge;   // the window's first code
            if (wi != run_w) {
                if (run) atomicAdd(&cnt[run_w], run);
                run_w = wi;
                run = 0;
            }
            ++run;
            // the code, first bit highest, at bit o of word k
            const uint64_t v = (uint64_t)code[e] << (64u - o - L);
            cur |= (uint32_t)(v >> 32);
            if (o + L >= 32) {
                if (first_word)   // (may hold the lane before's bits)
                    __hip_atomic_fetch_or(&a.stream[k], bswap32(cur), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else a.stream[k] = bswap32(cur);
                first_word = false;
                ++k;
                cur = (uint32_t)v;
                o = o + L - 32;
            } else {
                o += L;
            }
            pos += L;
            prev_len = L;
        });
        if (o)   // (may hold the next lane's bits)
            __hip_atomic_fetch_or(&a.stream[k], bswap32(cur), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (run) atomicAdd(&cnt[run_w], run);
        // raw bytes: (sign << 7) | fraction
        GLOBAL uint8_t *rb = a.raw + r.j0;
        uint32_t acc = 0;
        words.each([&](uint32_t i, uint32_t x) {
            acc |= (((x >> 8) & 0x80u) | (x & 0x7Fu)) << (8 * (i & 3));
            if ((i & 3) == 3) {
                *reinterpret_cast<GLOBAL uint32_t *>(rb + (i & ~3u)) = acc;
                acc = 0;
            }
        });
        if (r.m & 3) *reinterpret_cast<GLOBAL uint32_t *>(rb + (r.m & ~3u)) = acc;   // inside the 16-byte padding
    }
    __syncthreads();
    // the 512 window entries, cnt | gap << kWinGapShift, two per lane
    const uint32_t e0 = cnt[2 * tid] | (gap[2 * tid] << kWinGapShift);
    const uint32_t e1 = cnt[2 * tid + 1] | (gap[2 * tid + 1] << kWinGapShift);
    a.win[c * (kWindows / 2) + tid] = e0 | (e1 << 16);
}

// The 512-byte header, from a kernel argument (so that no host buffer has to
// outlive the call).
struct Header {
    uint32_t w[kHeader / 4];
};
__global__ __launch_bounds__(kHeader / 4) void enc_header(Header h, GLOBAL uint32_t *out) {
    out[threadIdx.x] = h.w[threadIdx.x];
}

}  // namespace

}  // namespace df11

using namespace df11;

extern "C" df11_status df11_encode_device_batch(int n_tensors, const void *const *d_words, const uint64_t *n_elems,
                                                const int *ndims, const uint64_t *dims, void *const *d_outs,
                                                const uint64_t *out_caps, uint64_t *out_bytes, int hip_device,
                                                hipStream_t stream) {
    if (n_tensors < 0 || (n_tensors && (!d_words || !n_elems || !ndims || !dims || !d_outs || !out_caps || !out_bytes)))
        return report_error(DF11_E_ARG, "df11_encode_device_batch: bad argument");
    for (int t = 0; t < n_tensors; ++t) {
        const uint64_t n = n_elems[t];
        const int ndim = ndims[t];
        if ((!d_words[t] && n) || !d_outs[t] || ndim < 0 || ndim > 8)
            return report_error(DF11_E_ARG, "df11_encode_device_batch: tensor %d: bad argument", t);
        uint64_t prod = 1;
        for (int i = 0; i < ndim; ++i) prod *= dims[8 * t + i];
        if ((ndim && prod != n) || (!ndim && n != 1))
            return report_error(DF11_E_ARG, "tensor %d: shape does not match %llu elements", t, (unsigned long long)n);
        if (n > (uint64_t(1) << 46)) return report_error(DF11_E_UNSUPPORTED, "tensor %d: %llu elements", t, (unsigned long long)n);
        if (((uintptr_t)d_words[t] & 15) || ((uintptr_t)d_outs[t] & 15))
            return report_error(DF11_E_ARG, "tensor %d: words and output must be 16-byte aligned", t);
        if (out_caps[t] < df11_container_bound(n))
            return report_error(DF11_E_ARG, "tensor %d: %llu bytes of output, below df11_container_bound (%llu)", t,
                                (unsigned long long)out_caps[t], (unsigned long long)df11_container_bound(n));
    }
    if (n_tensors == 0) return DF11_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(hip_device) != hipSuccess)
        return report_error(DF11_E_HIP, "df11_encode_device: device %d", hip_device);
    struct Restore {
        int d;
        ~Restore() { if (d >= 0) (void)hipSetDevice(d); }
    } restore{prev};
    auto hip_fail = [](hipError_t e, const char *what) {
        return report_error(DF11_E_HIP, "df11_encode_device: %s: %s", what, hipGetErrorString(e));
    };
    hipError_t e;

    // 1. every tensor's histogram, back to the host in one copy
    std::vector<uint64_t> freq((size_t)n_tensors * 256, 0);
    unsigned long long *hist = nullptr;
    const size_t hist_bytes = (size_t)n_tensors * 256 * sizeof(unsigned long long);
    if ((e = hipMallocAsync((void **)&hist, hist_bytes, stream)) != hipSuccess) return hip_fail(e, "hipMallocAsync");
    int n_cu = 0;
    (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, hip_device);
    e = hipMemsetAsync(hist, 0, hist_bytes, stream);
    for (int t = 0; t < n_tensors && e == hipSuccess; ++t) {
        if (!n_elems[t]) continue;
        const uint64_t need = (n_elems[t] + kEncThreads * 8 - 1) / (kEncThreads * 8);
        const int grid = (int)std::min<uint64_t>(need, (uint64_t)std::max(1, n_cu) * 8);
        hipLaunchKernelGGL(enc_hist, dim3(grid), dim3(kEncThreads), 0, stream, (const GLOBAL uint16_t *)d_words[t],
                           n_elems[t], (GLOBAL unsigned long long *)(hist + 256 * (size_t)t));
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpyAsync(freq.data(), hist, hist_bytes, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    const hipError_t ef = hipFreeAsync(hist, stream);
    if (e != hipSuccess) return hip_fail(e, "histogram");
    if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");

    // 2.-4. per tensor: the code, layout and header on the host; the header,
    // chunk bits, chunk index and packing enqueued (nothing waits for them)
    for (int t = 0; t < n_tensors; ++t) {
        const uint64_t n = n_elems[t];
        const uint64_t *f = freq.data() + 256 * (size_t)t;
        CodeTable T;
        build_code(f, T.len, T.code);
        uint64_t total_bits = 0;
        for (int sy = 0; sy < 256; ++sy) total_bits += f[sy] * T.len[sy];
        const EncodeLayout L = encode_layout(n, total_bits);
        Header h;
        write_header(reinterpret_cast<uint8_t *>(h.w), n, ndims[t], dims + 8 * t, L, T.len);
        uint8_t *out = static_cast<uint8_t *>(d_outs[t]);
        if ((e = hipMemsetAsync(out, 0, L.total, stream)) != hipSuccess) return hip_fail(e, "hipMemsetAsync");
        hipLaunchKernelGGL(enc_header, dim3(1), dim3(kHeader / 4), 0, stream, h, (GLOBAL uint32_t *)out);
        if (n) {
            const GLOBAL uint16_t *w = (const GLOBAL uint16_t *)d_words[t];
            GLOBAL uint64_t *ci = (GLOBAL uint64_t *)(out + L.off_ci);
            hipLaunchKernelGGL(enc_chunk_bits, dim3((unsigned)L.n_chunks), dim3(kEncThreads), 0, stream, w, n, T, ci);
            hipLaunchKernelGGL(enc_scan, dim3(1), dim3(kScanThreads), 0, stream, ci, L.n_chunks, n);
            PackArgs pa{w, n, ci, (GLOBAL uint32_t *)(out + L.off_stream), (GLOBAL uint32_t *)(out + L.off_win),
                        (GLOBAL uint8_t *)(out + L.off_raw)};
            hipLaunchKernelGGL(enc_pack, dim3((unsigned)L.n_chunks), dim3(kEncThreads), 0, stream, pa, T);
        }
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "launch");
        out_bytes[t] = L.total;
    }
    return DF11_OK;
}

extern "C" df11_status df11_encode_device(const void *d_words, uint64_t n, int ndim, const uint64_t *dims,
                                          void *d_out, uint64_t out_cap, uint64_t *out_bytes, int hip_device,
                                          hipStream_t stream) {
    if (!out_bytes || ndim < 0 || ndim > 8 || (ndim && !dims))
        return report_error(DF11_E_ARG, "df11_encode_device: bad argument");
    uint64_t d8[8] = {};
    for (int i = 0; i < ndim; ++i) d8[i] = dims[i];
    return df11_encode_device_batch(1, &d_words, &n, &ndim, d8, &d_out, &out_cap, out_bytes, hip_device, stream);
}
