// GPU encoder for gfx950: BF16 words in device memory -> version-4 container
// in device memory, byte for byte the container the host encoder writes.
//
// Method (mlx-dfloat project page, introduction and 16-bit weight diagram):
// each exponent byte gets a length-limited canonical prefix code, the sign +
// 7-bit fraction stay as one raw byte.  The df11pack page ("Measured")
// makes compression time the cost to cut; here the element-wise passes run
// on the GPU and only the 256-symbol code is built on the host:
//
//   1. histogram of the exponent byte per chunk (one read of the words),
//      kept where the chunk's window entries go later, and summed per tensor;
//   -- the host builds the code (package-merge, canonical values), the layout
//      from the total bit count sum(f * len), and the header;
//   2. per-chunk bit counts from the chunk histograms, written where the
//      chunk index goes;
//   3. one workgroup turns them into start bits (the chunk index) and
//      writes the header;
//   4. one 1024-lane workgroup per chunk: every lane packs the codes of 32
//      consecutive elements into 32-bit stream words, put together in LDS
//      and written out by the whole workgroup (the words a lane may share
//      with its neighbours with an OR), counts the codes that start in each
//      of the chunk's 512 windows and the offset of each window's first code
//      (in LDS), and writes the elements' raw bytes.  (1024 lanes of 32
//      elements measured 8% faster for the packing than 512 of 64.)
//
// Nothing is cleared before the kernels run: every byte of the container is
// written by one of them.  The stream words that take ORs in global memory
// (a chunk's first and last word, shared with the chunks before and after
// it) are cleared by the kernel of step 3, which also clears the gaps
// between and after the sections.
//
// The histogram is bound by its LDS atomics, the packing by its serial loop
// of 32 codes per lane; the words are read twice (2 bytes each) and about
// 1.36 bytes per element are written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "df11_internal.hpp"

namespace df11 {

// Histogram counters for the encoder entry point that allocates nothing:
// 256 per tensor, for at most kNoAllocTensors tensors per call (128 KiB).
// Each device holds its own copy until the process ends; host code reaches
// it only through the address hipGetSymbolAddress gives for that device
// (scratch_on below), never through this name.
constexpr int kNoAllocTensors = 64;
static __device__ __align__(256) unsigned long long scratch[kNoAllocTensors * 256];

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

constexpr int kEncThreads = 256;
constexpr int kPackThreads = 1024;                   // lanes per chunk in the packing kernel
constexpr int kPerLane = kChunk / kPackThreads;      // 32 elements per packing lane
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

// 1. exponent histogram, one workgroup per chunk: the chunk's 256 counts go
// to chunk_hist (u32 each, in the space the chunk's window entries take
// later) and are added into the tensor's u64 totals.  Bound by the LDS
// atomics once the loads are in flight together.
__global__ __launch_bounds__(kEncThreads) void enc_hist(const GLOBAL uint16_t *w, uint64_t n,
                                                        GLOBAL uint32_t *chunk_hist,
                                                        GLOBAL unsigned long long *hist) {
    // (each copy is one entry longer than the 256 bins, so that the copies of
    // a bin fall in different LDS banks; one copy per lane measured slower)
    __shared__ uint32_t h[kHistCopies][257];
    for (int i = threadIdx.x; i < kHistCopies * 257; i += kEncThreads) (&h[0][0])[i] = 0;
    __syncthreads();
    uint32_t *mine = h[threadIdx.x % kHistCopies];
    const uint64_t c = blockIdx.x;
    const uint64_t c0 = c * kChunk;
    const uint64_t cend = min(n, c0 + kChunk);
    if (cend - c0 == kChunk) {
        // a whole chunk: all 16 of a lane's 16-byte loads in flight before
        // their counts (one load, then its 8 counts, left the kernel waiting
        // on each load: 221 -> 174 us per Llama-8B block call)
        constexpr int kGroups = kChunk / (8 * kEncThreads);
        const GLOBAL u32x4 *src = reinterpret_cast<const GLOBAL u32x4 *>(w + c0) + threadIdx.x;
#pragma unroll
        for (int g = 0; g < kGroups; g += 16) {
            u32x4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = src[kEncThreads * (g + k)];
#pragma unroll
            for (int k = 0; k < 16; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i) atomicAdd(&mine[(word_of(v[k], i) >> 7) & 0xFFu], 1u);
        }
    } else
    for (uint64_t j = c0 + 8 * threadIdx.x; j < cend; j += 8 * kEncThreads) {
        if (j + 8 <= cend) {
            const u32x4 v = *reinterpret_cast<const GLOBAL u32x4 *>(w + j);
#pragma unroll
            for (int i = 0; i < 8; ++i) atomicAdd(&mine[(word_of(v, i) >> 7) & 0xFFu], 1u);
        } else {
            for (uint64_t k = j; k < cend; ++k) atomicAdd(&mine[(w[k] >> 7) & 0xFFu], 1u);
        }
    }
    __syncthreads();
    uint32_t sum = 0;
    for (int k = 0; k < kHistCopies; ++k) sum += h[(k + threadIdx.x) % kHistCopies][threadIdx.x];
    chunk_hist[c * 256 + threadIdx.x] = sum;
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
template <int N>
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t (&s)[2][N], uint32_t &total) {
    const uint32_t tid = threadIdx.x;
    s[0][tid] = v;
    __syncthreads();
    int src = 0;
    for (uint32_t d = 1; d < (uint32_t)N; d <<= 1) {
        const uint32_t x = s[src][tid] + (tid >= d ? s[src][tid - d] : 0u);
        s[src ^ 1][tid] = x;
        src ^= 1;
        __syncthreads();
    }
    total = s[src][N - 1];
    return s[src][tid] - v;
}

// 2. bits of each chunk, into the chunk index's start-bit slots: the sum of
// count x code length over the chunk's histogram (no second read of the
// words)
__global__ __launch_bounds__(kEncThreads) void enc_chunk_bits(const GLOBAL uint32_t *chunk_hist, CodeTable T,
                                                              GLOBAL uint64_t *ci) {
    __shared__ uint32_t s[2][kEncThreads];
    const uint64_t c = blockIdx.x;
    const uint32_t bits = chunk_hist[c * 256 + threadIdx.x] * (uint32_t)T.len[threadIdx.x];
    uint32_t total;
    block_exclusive(bits, s, total);
    if (threadIdx.x == 0) ci[2 * c] = total;
}

// The 512-byte header, from a kernel argument (so that no host buffer has to
// outlive the call), and the bytes no kernel writes otherwise: three ranges,
// 16-byte aligned, each a multiple of 16 bytes (the gaps after the chunk
// index and after the window entries, and the raw section's tail from the
// last group of 16 bytes the packing writes on).
struct Header {
    uint32_t w[kHeader / 4];
    uint64_t zero_at[3], zero_bytes[3];
};

// 3. start bits: exclusive prefix sum of the chunk bit counts, in place,
// with each chunk's first element and the sentinel {total bits, n}.  Then
// the stream words the packing ORs into are cleared (every other stream
// word it writes whole): each chunk's first and last word, which it may
// share with the chunks before and after it, and the section's padding
// after the last code (stream_words: the section's length in words).  The
// same workgroup writes the header and clears the gaps no kernel writes.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void enc_scan(GLOBAL uint64_t *ci, uint64_t n_chunks, uint64_t n,
                                                         GLOBAL uint32_t *stream, uint64_t stream_words,
                                                         Header h, GLOBAL uint32_t *out) {
    __shared__ uint64_t s[2][kScanThreads];
    __shared__ uint64_t carry;
    const uint32_t tid = threadIdx.x;
    // the header, and the gaps between and after the sections
    if (tid < kHeader / 4) out[tid] = h.w[tid];
    for (int r = 0; r < 3; ++r) {
        GLOBAL u32x4 *z = reinterpret_cast<GLOBAL u32x4 *>(reinterpret_cast<GLOBAL uint8_t *>(out) + h.zero_at[r]);
        for (uint64_t i = tid; i < h.zero_bytes[r] / 16; i += kScanThreads) z[i] = u32x4{0u, 0u, 0u, 0u};
    }
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
    // (every start bit was written before the last barrier; the total is in LDS)
    for (uint64_t c = tid; c < n_chunks; c += kScanThreads) {
        const uint64_t b = ci[2 * c], e = c + 1 < n_chunks ? ci[2 * c + 2] : carry;
        if (e > b) {
            stream[b >> 5] = 0u;
            stream[(e - 1) >> 5] = 0u;
        }
    }
    for (uint64_t k = ((carry + 31) >> 5) + tid; k < stream_words; k += kScanThreads) stream[k] = 0u;
}

struct PackArgs {
    const GLOBAL uint16_t *w;
    uint64_t n;
    const GLOBAL uint64_t *ci;   // the chunk index (start bits)
    GLOBAL uint32_t *stream;     // the stream section, zeroed, as 32-bit words
    GLOBAL uint32_t *win;        // the window section
    GLOBAL uint8_t *raw;         // the raw section
};

// A lane's words for its passes: held in registers when the lane has all 32
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

// 4. one chunk: codes into the stream, the window index, the raw bytes.
// The chunk's stream words are put together in LDS (a lane's words with
// plain writes, the two it may share with its neighbours with an LDS OR)
// and then written out by the whole workgroup, consecutive words across
// lanes; only the chunk's first and last words, which it may share with the
// chunks before and after it, take an atomic OR in global memory.  A chunk
// of more than kStageWords words (above 8 bits per element) is packed into
// global memory directly, with the same plain writes and ORs.
constexpr uint32_t kStageWords = 8192;

// A lane's codes into 32-bit stream words, first stream bit highest, its
// windows' counts and first-code offsets.  The lane's bits start at stream
// bit g0 (chunk bit p0); the codes go through a 64-bit register that holds
// the bits not yet written (the first word starts with the g0 % 32 bits of
// the lane before, as zeros), and every word that fills up is written out:
// staged chunks OR every word into the zeroed LDS words (the first and last
// may be shared with the neighbouring lanes), the others write plain words
// to global memory except the first and last, which they OR there.  A code
// whose start passes the next window edge takes the slow path: the window
// count so far goes out, and the new window's first-code offset is set.
template <bool kStaged>
__device__ __forceinline__ void pack_lane(const LaneWords &words, const uint32_t *tab, uint32_t *sw,
                                          GLOBAL uint32_t *stream, uint64_t k0, uint64_t g0, uint32_t p0,
                                          uint32_t N, uint32_t prev_len, uint32_t *cnt, uint32_t *gap) {
    uint64_t k = g0 >> 5;                  // the word being filled
    uint64_t acc = 0;                      // its bits so far, and any after
    uint32_t nb = (uint32_t)(g0 & 31);     // bits in acc not yet written
    bool first = true;
    auto put = [&](uint32_t v, bool shared) {
        if (kStaged) {
            atomicOr(&sw[k - k0], bswap32(v));   // (the LDS words start zero)
        } else if (shared) {
            __hip_atomic_fetch_or(&stream[k], bswap32(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            stream[k] = bswap32(v);
        }
    };
    // the window of the lane's first code: the last one whose edge is at or
    // before it (windows start at floor(i N / 512))
    uint32_t wi = min((uint32_t)kWindows - 1u, (kWindows * (p0 + 1u) - 1u) / N);
    uint32_t next_edge = wi + 1u < (uint32_t)kWindows ? window_edge(N, wi + 1u) : ~0u;
    if (p0 == 0 || window_edge(N, wi) > p0 - prev_len) gap[wi] = p0 - window_edge(N, wi);
    uint32_t run = 0;
    uint32_t pos = p0;
    words.each([&](uint32_t, uint32_t x) {
        const uint32_t ent = tab[(x >> 7) & 0xFFu];
        const uint32_t L = ent & 0xFFu;
        if (pos >= next_edge) {
            // the first code to start in a later window (the windows passed
            // over hold no code start)
            atomicAdd(&cnt[wi], run);
            run = 0;
            do {
                ++wi;
            } while (wi + 1u < (uint32_t)kWindows && window_edge(N, wi + 1u) <= pos);
            gap[wi] = pos - window_edge(N, wi);
            next_edge = wi + 1u < (uint32_t)kWindows ? window_edge(N, wi + 1u) : ~0u;
        }
        ++run;
        pos += L;
        acc = (acc << L) | (ent >> 8);
        nb += L;
        if (nb >= 32u) {
            nb -= 32u;
            put((uint32_t)(acc >> nb), first);
            first = false;
            ++k;
        }
    });
    if (nb) put((uint32_t)(acc << (32u - nb)), true);   // (shared with the lane after)
    if (run) atomicAdd(&cnt[wi], run);
}

// The raw bytes, (sign << 7) | fraction, of a lane holding all its words:
// four at a time from two words of the 16-byte groups (masks, shifts and
// one byte permute), 16 bytes per store.
__device__ __forceinline__ uint32_t raw4(uint32_t d0, uint32_t d1) {
    const uint32_t t0 = (d0 & 0x007F007Fu) | ((d0 >> 8) & 0x00800080u);
    const uint32_t t1 = (d1 & 0x007F007Fu) | ((d1 >> 8) & 0x00800080u);
    return __builtin_amdgcn_perm(t1, t0, 0x06040200u);
}

__global__ __launch_bounds__(kPackThreads) void enc_pack(PackArgs a, CodeTable T) {
    __shared__ uint32_t tab[256];          // code << 8 | length
    __shared__ uint32_t cnt[kWindows], gap[kWindows];
    __shared__ uint32_t s[2][kPackThreads];
    __shared__ uint8_t last_len[kPackThreads];
    __shared__ uint32_t sw[kStageWords];
    const uint32_t tid = threadIdx.x;
    const uint64_t c = blockIdx.x;
    if (tid < 256) tab[tid] = (T.code[tid] << 8) | T.len[tid];
    static_assert(kWindows / 2 <= kPackThreads, "two window entries per lane");
    static_assert(kMaxLen <= 24, "code << 8 fits 32 bits");
    for (uint32_t i = tid; i < (uint32_t)kWindows; i += kPackThreads) {
        cnt[i] = 0;
        gap[i] = 0;
    }
    const uint64_t b0 = a.ci[2 * c];
    const uint32_t N = (uint32_t)(a.ci[2 * c + 2] - b0);   // the chunk's bits
    const uint64_t k0 = b0 >> 5;                            // its first stream word
    const uint32_t nw = N ? (uint32_t)(((b0 + N - 1) >> 5) - k0 + 1) : 0u;
    const bool staged = nw <= kStageWords;
    if (staged)
        for (uint32_t i = tid; i < nw; i += kPackThreads) sw[i] = 0u;
    __syncthreads();

    const LaneRange r = lane_range(c, tid, a.n);
    const LaneWords words(a.w, r);
    // this lane's bits and its last element's code length, for its neighbours
    uint32_t bits = 0, lastl = 0;
    words.each([&](uint32_t, uint32_t x) {
        lastl = tab[(x >> 7) & 0xFFu] & 0xFFu;
        bits += lastl;
    });
    last_len[tid] = (uint8_t)lastl;
    uint32_t nbits_scan;
    const uint32_t p0 = block_exclusive(bits, s, nbits_scan);   // (its barriers publish last_len)
    // A chunk packed straight into global memory: the words its lanes OR into
    // (each lane's first word and its last, partial one, which it may share
    // with its neighbours) are cleared first, except the chunk's own first
    // and last words, which the scan kernel cleared and the chunks before and
    // after OR into as well.  The clearing takes atomics, as the ORs do, and
    // is complete (fence, barrier) before any lane ORs.
    if (!staged) {
        if (bits) {
            const uint64_t g0 = b0 + p0, g1 = g0 + bits;   // the lane's stream bits [g0, g1)
            const uint64_t kf = g0 >> 5, kl = (g1 - 1) >> 5, kc1 = k0 + nw - 1;
            if (kf != k0 && kf != kc1)
                __hip_atomic_exchange(&a.stream[kf], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((g1 & 31u) && kl != kf && kl != k0 && kl != kc1)
                __hip_atomic_exchange(&a.stream[kl], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __threadfence();
        __syncthreads();
    }

    if (r.m) {
        const uint32_t prev_len = tid ? last_len[tid - 1] : 0u;   // the code before the lane's first
        if (staged)
            pack_lane<true>(words, tab, sw, a.stream, k0, b0 + p0, p0, N, prev_len, cnt, gap);
        else
            pack_lane<false>(words, tab, sw, a.stream, k0, b0 + p0, p0, N, prev_len, cnt, gap);
        // raw bytes: (sign << 7) | fraction, 16 at a time (a partial last
        // group inside the section's 16-byte padding, its missing bytes zero)
        GLOBAL uint8_t *rb = a.raw + r.j0;
        if (words.full) {
#pragma unroll
            for (int g = 0; g < kPerLane / 8; g += 2) {
                const u32x4 &v = words.v[g], &u = words.v[g + 1];
                *reinterpret_cast<GLOBAL u32x4 *>(rb + 8 * g) =
                    u32x4{raw4(v.x, v.y), raw4(v.z, v.w), raw4(u.x, u.y), raw4(u.z, u.w)};
            }
        } else {
            u32x4 acc{0u, 0u, 0u, 0u};
            words.each([&](uint32_t i, uint32_t x) {
                const uint32_t b = (((x >> 8) & 0x80u) | (x & 0x7Fu)) << (8 * (i & 3));
                const uint32_t q = (i >> 2) & 3u;
                acc.x |= q == 0 ? b : 0u;
                acc.y |= q == 1 ? b : 0u;
                acc.z |= q == 2 ? b : 0u;
                acc.w |= q == 3 ? b : 0u;
                if ((i & 15) == 15) {
                    *reinterpret_cast<GLOBAL u32x4 *>(rb + (i & ~15u)) = acc;
                    acc = u32x4{0u, 0u, 0u, 0u};
                }
            });
            if (r.m & 15) *reinterpret_cast<GLOBAL u32x4 *>(rb + (r.m & ~15u)) = acc;
        }
    }
    __syncthreads();
    // the staged words, consecutive across lanes; the chunk's first and last
    // words are ORed (the chunks before and after may have bits in them)
    if (staged) {
        for (uint32_t i = tid; i < nw; i += kPackThreads) {
            const uint32_t v = sw[i];
            if (i == 0 || i == nw - 1)
                __hip_atomic_fetch_or(&a.stream[k0 + i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                a.stream[k0 + i] = v;
        }
    }
    // the 512 window entries, cnt | gap << kWinGapShift, two per lane of the
    // first 256
    if (tid < kWindows / 2) {
        const uint32_t e0 = cnt[2 * tid] | (gap[2 * tid] << kWinGapShift);
        const uint32_t e1 = cnt[2 * tid + 1] | (gap[2 * tid + 1] << kWinGapShift);
        a.win[c * (kWindows / 2) + tid] = e0 | (e1 << 16);
    }
}

// Zeroes n counters (the histograms, before they are counted).
__global__ __launch_bounds__(kEncThreads) void enc_clear(GLOBAL unsigned long long *p, uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * kEncThreads + threadIdx.x;
    if (i < n) p[i] = 0;
}

constexpr int kMaxDevices = 64;
// Guards scratch_ptr, the host copy of the counts and every use of a
// device's scratch: calls of the no-alloc entry point take turns.
std::mutex g_scratch_mu;
unsigned long long *g_scratch_ptr[kMaxDevices];
uint64_t g_freq[kNoAllocTensors * 256];

// This device's scratch (hipGetSymbolAddress once per device, with the
// device current; called with g_scratch_mu held).
hipError_t scratch_on(int device, unsigned long long **ptr) {
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = static_cast<unsigned long long *>(p);
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

df11_status check_batch(const char *who, int n_tensors, const void *const *d_words, const uint64_t *n_elems,
                        const int *ndims, const uint64_t *dims, void *const *d_outs, const uint64_t *out_caps,
                        uint64_t *out_bytes) {
    if (n_tensors < 0 || (n_tensors && (!d_words || !n_elems || !ndims || !dims || !d_outs || !out_caps || !out_bytes)))
        return report_error(DF11_E_ARG, "%s: bad argument", who);
    for (int t = 0; t < n_tensors; ++t) {
        const uint64_t n = n_elems[t];
        const int ndim = ndims[t];
        if ((!d_words[t] && n) || !d_outs[t] || ndim < 0 || ndim > 8)
            return report_error(DF11_E_ARG, "%s: tensor %d: bad argument", who, t);
        uint64_t prod = 1;
        for (int i = 0; i < ndim; ++i) prod *= dims[8 * t + i];
        if ((ndim && prod != n) || (!ndim && n != 1))
            return report_error(DF11_E_ARG, "%s: tensor %d: shape does not match %llu elements", who, t,
                                (unsigned long long)n);
        if (n > (uint64_t(1) << 46))
            return report_error(DF11_E_UNSUPPORTED, "%s: tensor %d: %llu elements", who, t, (unsigned long long)n);
        if (((uintptr_t)d_words[t] & 15) || ((uintptr_t)d_outs[t] & 15))
            return report_error(DF11_E_ARG, "%s: tensor %d: words and output must be 16-byte aligned", who, t);
        if (out_caps[t] < df11_container_bound(n))
            return report_error(DF11_E_ARG, "%s: tensor %d: %llu bytes of output, below df11_container_bound (%llu)",
                                who, t, (unsigned long long)out_caps[t], (unsigned long long)df11_container_bound(n));
    }
    return DF11_OK;
}

// Makes hip_device current for the caller's scope and puts the previous one
// back.
struct DeviceScope {
    int prev = -1;
    bool ok = false;
    explicit DeviceScope(int dev) {
        ok = hipGetDevice(&prev) == hipSuccess && hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceScope() {
        if (ok && prev >= 0) (void)hipSetDevice(prev);
    }
};

df11_status hip_fail(const char *who, hipError_t e, const char *what) {
    return report_error(DF11_E_HIP, "%s: %s: %s", who, what, hipGetErrorString(e));
}

// 1. every tensor's exponent histogram into hist (256 counters per tensor,
// cleared here), then back to the host (freq) in one copy; waits for it.
// Where a tensor's per-chunk histograms wait between the histogram and the
// chunk bits: the container's window section, n_chunks x 1 KiB (the packing
// overwrites it), whose offset depends on the element count only.
GLOBAL uint32_t *chunk_hist_of(void *d_out, uint64_t n) {
    const EncodeLayout L = encode_layout(n, 0);
    return (GLOBAL uint32_t *)(static_cast<uint8_t *>(d_out) + L.off_win);
}
static_assert(kWindows * 2 == 256 * sizeof(uint32_t), "a chunk's histogram fills its window entries");

hipError_t histograms(int n_tensors, const void *const *d_words, const uint64_t *n_elems, void *const *d_outs,
                      unsigned long long *hist, uint64_t *freq, hipStream_t stream) {
    const uint64_t n_ctr = (uint64_t)n_tensors * 256;
    hipLaunchKernelGGL(enc_clear, dim3((unsigned)((n_ctr + kEncThreads - 1) / kEncThreads)), dim3(kEncThreads), 0,
                       stream, (GLOBAL unsigned long long *)hist, n_ctr);
    hipError_t e = hipGetLastError();
    for (int t = 0; t < n_tensors && e == hipSuccess; ++t) {
        if (!n_elems[t]) continue;
        const uint64_t n_chunks = (n_elems[t] + kChunk - 1) / kChunk;
        hipLaunchKernelGGL(enc_hist, dim3((unsigned)n_chunks), dim3(kEncThreads), 0, stream,
                           (const GLOBAL uint16_t *)d_words[t], n_elems[t], chunk_hist_of(d_outs[t], n_elems[t]),
                           (GLOBAL unsigned long long *)(hist + 256 * (size_t)t));
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpyAsync(freq, hist, n_ctr * sizeof(unsigned long long), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return e;
}

// 2.-4. per tensor: the code, layout and header on the host; the header,
// chunk bits, chunk index and packing enqueued (nothing waits for them).
df11_status pack_batch(const char *who, int n_tensors, const void *const *d_words, const uint64_t *n_elems,
                       const int *ndims, const uint64_t *dims, void *const *d_outs, uint64_t *out_bytes,
                       const uint64_t *freq, hipStream_t stream) {
    hipError_t e;
    for (int t = 0; t < n_tensors; ++t) {
        const uint64_t n = n_elems[t];
        const uint64_t *f = freq + 256 * (size_t)t;
        CodeTable T;
        build_code(f, T.len, T.code);
        uint64_t total_bits = 0;
        for (int sy = 0; sy < 256; ++sy) total_bits += f[sy] * T.len[sy];
        const EncodeLayout L = encode_layout(n, total_bits);
        Header h;
        write_header(reinterpret_cast<uint8_t *>(h.w), n, ndims[t], dims + 8 * t, L, T.len);
        uint8_t *out = static_cast<uint8_t *>(d_outs[t]);
        // the kernels write the header, the chunk index, the window entries,
        // the stream (clearing the words they OR into themselves) and the raw
        // bytes (up to the 16 bytes holding element n - 1); clear the rest:
        // the gaps after the chunk index and the window entries, and the raw
        // section's tail padding
        // (an empty tensor: all of it after the header is cleared)
        const uint64_t ci_end = n ? L.off_ci + (L.n_chunks + 1) * 16 : kHeader;
        const uint64_t win_end = L.off_win + L.n_chunks * kWindows * 2;
        const uint64_t stream_at = n ? L.off_stream : L.off_raw;
        const uint64_t raw_set = L.off_raw + (n & ~uint64_t(15));
        h.zero_at[0] = ci_end;
        h.zero_bytes[0] = L.off_win - ci_end;
        h.zero_at[1] = win_end;
        h.zero_bytes[1] = stream_at - win_end;
        h.zero_at[2] = raw_set;
        h.zero_bytes[2] = L.total - raw_set;
        GLOBAL uint64_t *ci = (GLOBAL uint64_t *)(out + L.off_ci);
        if (n)
            hipLaunchKernelGGL(enc_chunk_bits, dim3((unsigned)L.n_chunks), dim3(kEncThreads), 0, stream,
                               (const GLOBAL uint32_t *)chunk_hist_of(out, n), T, ci);
        // (an empty tensor: the header and its zero chunk index entry, the
        // rest cleared)
        hipLaunchKernelGGL(enc_scan, dim3(1), dim3(kScanThreads), 0, stream, ci, L.n_chunks, n,
                           (GLOBAL uint32_t *)(out + (n ? L.off_stream : L.off_raw)),
                           n ? (L.off_raw - L.off_stream) / 4 : 0, h, (GLOBAL uint32_t *)out);
        if (n) {
            const GLOBAL uint16_t *w = (const GLOBAL uint16_t *)d_words[t];
            PackArgs pa{w, n, ci, (GLOBAL uint32_t *)(out + L.off_stream), (GLOBAL uint32_t *)(out + L.off_win),
                        (GLOBAL uint8_t *)(out + L.off_raw)};
            hipLaunchKernelGGL(enc_pack, dim3((unsigned)L.n_chunks), dim3(kPackThreads), 0, stream, pa, T);
        }
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(who, e, "launch");
        out_bytes[t] = L.total;
    }
    return DF11_OK;
}

}  // namespace

}  // namespace df11

using namespace df11;

extern "C" df11_status df11_encode_device_batch(int n_tensors, const void *const *d_words, const uint64_t *n_elems,
                                                const int *ndims, const uint64_t *dims, void *const *d_outs,
                                                const uint64_t *out_caps, uint64_t *out_bytes, int hip_device,
                                                hipStream_t stream) {
    const char *who = "df11_encode_device_batch";
    df11_status st = check_batch(who, n_tensors, d_words, n_elems, ndims, dims, d_outs, out_caps, out_bytes);
    if (st != DF11_OK || n_tensors == 0) return st;
    DeviceScope scope(hip_device);
    if (!scope.ok) return report_error(DF11_E_HIP, "%s: device %d", who, hip_device);
    std::vector<uint64_t> freq((size_t)n_tensors * 256, 0);
    unsigned long long *hist = nullptr;
    hipError_t e = hipMallocAsync((void **)&hist, (size_t)n_tensors * 256 * sizeof(unsigned long long), stream);
    if (e != hipSuccess) return hip_fail(who, e, "hipMallocAsync");
    e = histograms(n_tensors, d_words, n_elems, d_outs, hist, freq.data(), stream);
    const hipError_t ef = hipFreeAsync(hist, stream);
    if (e != hipSuccess) return hip_fail(who, e, "histogram");
    if (ef != hipSuccess) return hip_fail(who, ef, "hipFreeAsync");
    return pack_batch(who, n_tensors, d_words, n_elems, ndims, dims, d_outs, out_bytes, freq.data(), stream);
}

extern "C" df11_status df11_encode_device_batch_noalloc(int n_tensors, const void *const *d_words,
                                                        const uint64_t *n_elems, const int *ndims,
                                                        const uint64_t *dims, void *const *d_outs,
                                                        const uint64_t *out_caps, uint64_t *out_bytes,
                                                        int hip_device, hipStream_t stream) {
    const char *who = "df11_encode_device_batch_noalloc";
    if (n_tensors > kNoAllocTensors)
        return report_error(DF11_E_UNSUPPORTED, "%s: %d tensors, at most %d per call", who, n_tensors,
                            kNoAllocTensors);
    if (hip_device < 0 || hip_device >= kMaxDevices)
        return report_error(DF11_E_ARG, "%s: device %d", who, hip_device);
    df11_status st = check_batch(who, n_tensors, d_words, n_elems, ndims, dims, d_outs, out_caps, out_bytes);
    if (st != DF11_OK || n_tensors == 0) return st;
    DeviceScope scope(hip_device);
    if (!scope.ok) return report_error(DF11_E_HIP, "%s: device %d", who, hip_device);
    std::lock_guard<std::mutex> hold(g_scratch_mu);
    unsigned long long *hist = nullptr;
    hipError_t e = scratch_on(hip_device, &hist);
    if (e != hipSuccess) return hip_fail(who, e, "hipGetSymbolAddress");
    if ((e = histograms(n_tensors, d_words, n_elems, d_outs, hist, g_freq, stream)) != hipSuccess)
        return hip_fail(who, e, "histogram");
    return pack_batch(who, n_tensors, d_words, n_elems, ndims, dims, d_outs, out_bytes, g_freq, stream);
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
