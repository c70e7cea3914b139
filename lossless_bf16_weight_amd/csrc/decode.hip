// DFloat11-style decode kernel for gfx950 (CDNA4).
//
// Method (mlx-dfloat project page, introduction and 16-bit weight diagram):
// each BF16 weight is rebuilt from its raw byte (sign << 7 | 7-bit fraction)
// and its exponent byte, which is stored as a variable-length prefix code in
// one bitstream; output words are bit-identical to the originals.
//
// One workgroup = one wave64.  A wave decodes whole chunks of 32768 elements
// (64 KiB of BF16 output), one after the other, over a contiguous range of
// the launch's work items (tensor, chunk):
//
//   1. stage: coalesced 16-byte loads of the chunk's code bytes, byte-swapped
//      into big-endian 32-bit words in LDS; the chunk's raw bytes are loaded
//      into registers at the same time (8 bytes per lane per half-block) and
//      are not needed before step 5, so their latency hides behind decoding;
//   2. index: each lane reads its window's (gap, cnt); a DPP prefix sum over
//      the 64 counts gives every lane the chunk position of its first code;
//   3. decode: each lane walks its window with a 64-bit bit buffer; one look-up
//      in the LDS first-level table resolves up to three codes of <= 10 bits;
//      longer codes go through the canonical limit table.  Exponent bytes are
//      OR-ed into a zeroed 32 KiB LDS tile at their chunk positions;
//   4. check: a lane must end exactly where the next non-empty window's first
//      code starts (or at the chunk end); otherwise the plan's flag is set;
//   5. assemble: per 1024 elements, each lane joins 2 x 8 exponents from the
//      tile with 2 x 8 raw bytes into BF16 words -- (r & 0x80) << 8 |
//      e << 7 | (r & 0x7F) -- and writes them with two 16-byte stores that are
//      contiguous across the wave (1 KiB per store instruction).
//
// There is no matrix arithmetic here: the path is bound by HBM traffic
// (about 1.33 bytes read and 2 bytes written per element), with integer
// ALU and LDS issue as the secondary limit.
#include <hip/hip_runtime.h>

#include "df11_internal.hpp"

namespace df11 {

constexpr int kTileBytes = kChunk;                 // one exponent byte per element
constexpr int kCodeCap = 15 * 1024;                // staged code bytes per chunk
constexpr int kCodeWords = kCodeCap / 4;
constexpr int kBlocks = kChunk / 1024;             // 1024-element blocks per chunk

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Lds {
    uint32_t tile[kTileBytes / 4 + 4];
    uint32_t codes[kCodeWords];
    LutRecord lut;
};

__device__ __forceinline__ uint32_t bswap32(uint32_t x) {
    return __builtin_amdgcn_perm(0u, x, 0x00010203u);
}

// Inclusive prefix sum over the 64 lanes of the wave, with DPP row shifts
// inside each row of 16 lanes and row broadcasts between rows.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// BF16 words of two elements from their exponents and raw bytes, packed.
__device__ __forceinline__ uint32_t join2(uint32_t e01, uint32_t r01) {
    // x = [e1 r1 e0 r0] (bytes from high to low): each half is (e << 8) | r
    const uint32_t x = __builtin_amdgcn_perm(e01, r01, 0x05010400u);
    // half -> (r & 0x80) << 8 | e << 7 | (r & 0x7F)
    return (x & 0x007F007Fu) | ((x >> 1) & 0x7F807F80u) | ((x << 8) & 0x80008000u);
}

__device__ __forceinline__ u32x4 join8(u32x2 e8, u32x2 r8) {
    u32x4 o;
    o.x = join2(e8.x, r8.x);
    o.y = join2(e8.x >> 16, r8.x >> 16);
    o.z = join2(e8.y, r8.y);
    o.w = join2(e8.y >> 16, r8.y >> 16);
    return o;
}

// Decode `rem` codes starting at relative bit `s` of `words` (big-endian
// 32-bit words, clamped to `n_words`), OR-ing the exponent bytes into the
// tile from byte position `q`.  Returns the relative bit after the last code.
template <bool kFromLds>
__device__ __forceinline__ uint64_t decode_window(Lds &L, const uint32_t *__restrict__ words,
                                                  uint32_t n_words, uint64_t s, uint32_t q,
                                                  uint32_t rem, uint32_t &bad) {
    auto word = [&](uint64_t i) -> uint32_t {
        const uint64_t j = i < n_words ? i : (uint64_t)n_words - 1;
        if constexpr (kFromLds) return words[j];
        else return bswap32(words[j]);
    };
    uint64_t rd = s >> 5;
    const uint32_t sh = (uint32_t)(s & 31);
    uint64_t buf = (((uint64_t)word(rd) << 32) | word(rd + 1)) << sh;
    int nb = 64 - (int)sh;
    rd += 2;
    uint32_t nxt = word(rd);
    while (rem > 0) {
        const uint32_t top = (uint32_t)(buf >> 32);
        const uint32_t ent = L.lut.l1[top >> (32 - kL1Bits)];
        uint32_t n = ent >> 28;
        uint32_t c = (ent >> 24) & 15u;
        uint32_t syms = ent & 0xFFFFFFu;
        if (n == 0) {
            // a code longer than kL1Bits: canonical limits, 24-bit peek
            const uint32_t v = top >> 8;
            int l = kL1Bits + 1;
            while (l <= kMaxLen && v >= L.lut.lim[l]) ++l;
            if (l > kMaxLen) {
                bad = 1;
                l = kMaxLen;
                syms = 0;
            } else {
                syms = L.lut.sorted[(int)(v >> (kMaxLen - l)) + L.lut.base[l]];
            }
            n = 1;
            c = (uint32_t)l;
        }
        if (n > rem) {
            // last look-up of the window: keep only its first `rem` codes
            n = rem;
            c = 0;
            for (uint32_t k = 0; k < n; ++k) c += L.lut.len[(syms >> (8 * k)) & 0xFFu];
            syms &= (1u << (8 * n)) - 1u;
        }
        const uint64_t v64 = (uint64_t)syms << (8 * (q & 3));
        __hip_atomic_fetch_or(&L.tile[q >> 2], (uint32_t)v64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_or(&L.tile[(q >> 2) + 1], (uint32_t)(v64 >> 32), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
        q += n;
        rem -= n;
        buf <<= c;
        nb -= (int)c;
        if (nb <= 32) {
            buf |= (uint64_t)nxt << (32 - nb);
            nb += 32;
            ++rd;
            nxt = word(rd);
        }
    }
    return rd * 32 - (uint64_t)nb;
}

__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
    __shared__ Lds L;
    const uint32_t lane = threadIdx.x;
    const uint32_t begin = (uint32_t)((uint64_t)a.n_items * blockIdx.x / gridDim.x);
    const uint32_t end = (uint32_t)((uint64_t)a.n_items * (blockIdx.x + 1) / gridDim.x);
    uint32_t cur_lut = 0xFFFFFFFFu;
    uint32_t bad_any = 0;

    for (uint32_t item = begin; item < end; ++item) {
        uint32_t tl, chunk;
        if (a.work) {
            const uint32_t w = a.work[item];
            tl = w >> kItemChunkBits;
            chunk = w & kItemChunkMask;
        } else {
            tl = 0;
            chunk = item;
        }
        const TensorDesc &d = a.desc[a.tensor_base + tl];
        const uint8_t *__restrict__ C = a.containers[tl];
        uint16_t *__restrict__ out = a.outs[tl];
        const uint64_t n_elems = d.n_elems;
        const uint64_t elem0 = (uint64_t)chunk * kChunk;
        const uint32_t nc = (uint32_t)min<uint64_t>(kChunk, n_elems - elem0);

        // ---- decode tables of this tensor -> LDS
        if (d.lut_index != cur_lut) {
            __syncthreads();
            const u32x4 *src = reinterpret_cast<const u32x4 *>(a.luts + d.lut_index);
            u32x4 *dst = reinterpret_cast<u32x4 *>(&L.lut);
            for (uint32_t i = lane; i < sizeof(LutRecord) / 16; i += 64) dst[i] = src[i];
            cur_lut = d.lut_index;
        }

        // ---- chunk index
        const uint64_t *ci = reinterpret_cast<const uint64_t *>(C + d.off_ci) + 2 * (uint64_t)chunk;
        const uint64_t b0 = ci[0];
        const uint64_t b1 = max(ci[2], b0);
        const uint32_t gap = C[d.off_gap + (uint64_t)chunk * kLanes + lane];
        const uint32_t cnt = reinterpret_cast<const uint16_t *>(C + d.off_cnt)[(uint64_t)chunk * kLanes + lane];

        // ---- stage the code bytes (16-byte aligned window) and prefetch raw
        const uint8_t *stream = C + d.off_stream;
        const uint64_t sbytes = d.stream_bytes;
        const uint64_t s0 = min<uint64_t>((b0 >> 3) & ~(uint64_t)15, sbytes - 16);
        const uint64_t s_end = min<uint64_t>((((b1 + 127) >> 3) + 15) & ~(uint64_t)15, sbytes);
        const bool staged = s_end <= s0 + kCodeCap;

        u32x4 cw[kCodeCap / 1024];
        if (staged) {
#pragma unroll
            for (int k = 0; k < kCodeCap / 1024; ++k) {
                const uint64_t off = min<uint64_t>(s0 + 1024 * k + 16 * lane, sbytes - 16);
                cw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(stream + off));
            }
        }
        const uint8_t *raw = C + d.off_raw;
        const uint64_t raw_last = d.raw_bytes - 8;
        u32x2 rw[2 * kBlocks];
#pragma unroll
        for (int b = 0; b < 2 * kBlocks; ++b) {
            const uint64_t j = min<uint64_t>(elem0 + 512 * b + 8 * lane, raw_last);
            rw[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(raw + j));
        }

        // ---- zero the tile; write the staged words
        __syncthreads();
        {
            u32x4 *t4 = reinterpret_cast<u32x4 *>(L.tile);
            for (uint32_t i = lane; i < sizeof(L.tile) / 16; i += 64) t4[i] = u32x4{0, 0, 0, 0};
        }
        if (staged) {
#pragma unroll
            for (int k = 0; k < kCodeCap / 1024; ++k) {
                u32x4 v = cw[k];
                v.x = bswap32(v.x);
                v.y = bswap32(v.y);
                v.z = bswap32(v.z);
                v.w = bswap32(v.w);
                reinterpret_cast<u32x4 *>(L.codes)[64 * k + lane] = v;
            }
        }

        // ---- lane windows: first code position and output position
        const uint64_t W = (b1 - b0 + kLanes - 1) / kLanes;
        const uint32_t incl = wave_inclusive_sum(cnt);
        const uint32_t q0 = incl - cnt;
        // never write past the tile, whatever the device bytes say
        uint32_t rem = q0 < nc ? min(cnt, nc - q0) : 0u;
        const uint64_t start = b0 + lane * W + (cnt ? gap : 0u);
        __syncthreads();

        uint32_t bad = 0;
        uint64_t stop = start;
        if (rem > 0) {
            if (staged) {
                stop = decode_window<true>(L, L.codes, kCodeWords, start - 8 * s0, q0, rem, bad) + 8 * s0;
            } else {
                stop = decode_window<false>(L, reinterpret_cast<const uint32_t *>(stream),
                                            (uint32_t)(sbytes / 4), start, q0, rem, bad);
            }
        }

        // ---- each non-empty window must end where the next one's first code
        //      starts, the last one at the chunk end
        const uint64_t mask = __ballot(cnt != 0);
        const uint64_t next_start = __shfl_down((unsigned long long)start, 1);
        const uint64_t above = lane == 63 ? 0 : (mask >> (lane + 1));
        if (cnt != 0) {
            if (above == 0) bad |= stop != b1;
            else if (above & 1) bad |= stop != next_start;
        }
        if (rem != cnt) bad = 1;
        bad_any |= bad;
        __syncthreads();

        // ---- assemble and store
        uint16_t *o = out + elem0;
#pragma unroll
        for (int b = 0; b < 2 * kBlocks; ++b) {
            const uint32_t j = 512 * b + 8 * lane;
            if (512u * b >= nc) break;
            const u32x2 e8 = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint8_t *>(L.tile) + j);
            const u32x4 v = join8(e8, rw[b]);
            if (j + 8 <= nc) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(o + j));
            } else if (j < nc) {
                const uint32_t part[4] = {v.x, v.y, v.z, v.w};
                for (uint32_t k = 0; j + k < nc; ++k) o[j + k] = (uint16_t)(part[k >> 1] >> (16 * (k & 1)));
            }
        }
    }
    if (__ballot(bad_any) && lane == 0) atomicOr(a.status, 1u);
}

hipError_t launch_decode(const DecodeArgs &args, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(64), 0, stream, args);
    return hipGetLastError();
}

int decode_wgs_per_cu() {
    static int cached = 0;
    if (!cached) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel, 64, 0) != hipSuccess || n <= 0) n = 1;
        cached = n;
    }
    return cached;
}

}  // namespace df11
