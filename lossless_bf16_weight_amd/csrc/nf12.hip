// NF12 decode kernel for gfx950: the fixed-rate 12-bit format (nf12 news
// page, "Developer open-sources nf12: lossless 12-bit compression for BF16
// models", "How it works" and "Implementation details").
//
// A group of 8 weights whose top four exponent bits are all 0111 is stored as
// 8 codes of 12 bits in 12 bytes, code i = (sign << 11) | (low four exponent
// bits << 7) | fraction at bits 12i .. 12i+11; every other group is flagged
// in a bitmap and its 8 words sit whole in an escape buffer, in group order.
//
// One lane per group: a wave takes the 64 groups of one bitmap word (768
// bytes in, 1 KiB out, both contiguous), so an outlier finds its escape entry
// from the word's prefix count plus a popcount of the flags below its lane.
// A launch decodes up to kNf12MaxBatch tensors: their bitmap words form one
// range, which workgroups sweep block-cyclically with four words per wave in
// flight, like the bandwidth control, since the path is bound by HBM
// traffic: 12 bytes read and 16 written per 8 weights (plus 16 escape bytes
// for an outlier group).
#include <hip/hip_runtime.h>

#include "nf12_internal.hpp"

namespace df11 {

namespace {

constexpr int kNfThreads = 256;
constexpr int kNfUnroll = 4;

typedef uint32_t v3u __attribute__((ext_vector_type(3)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// The word of a 12-bit code: the top four exponent bits are 0111 again.
__device__ __forceinline__ uint32_t nf12_word(uint32_t c) {
    return ((c & 0x800u) << 4) | 0x3800u | (c & 0x7FFu);
}

__device__ __forceinline__ uint32_t pair(uint32_t lo, uint32_t hi) {
    return nf12_word(lo & 0xFFFu) | (nf12_word(hi & 0xFFFu) << 16);
}

// The 8 words of a group from its 12 bytes (d.x = bits 0..31 of the group).
__device__ __forceinline__ v4u expand(v3u d) {
    return v4u{pair(d.x, d.x >> 12),
               pair(__builtin_amdgcn_alignbit(d.y, d.x, 24), d.y >> 4),
               pair(d.y >> 16, __builtin_amdgcn_alignbit(d.z, d.y, 28)),
               pair(d.z >> 8, d.z >> 20)};
}

// Moves t to the tensor of the launch that bitmap word w belongs to.  A
// wave meets its words in increasing order, so the scan resumes where it
// stopped (uniform per wave, in scalar registers).
__device__ __forceinline__ void advance_to(const Nf12Args &a, uint64_t w, uint32_t &t) {
    while (t + 1 < a.n_tensors && a.t[t + 1].word_base <= w) ++t;
}

__global__ __launch_bounds__(kNfThreads) void nf12_decode_kernel(Nf12Args a) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    constexpr uint32_t kWaves = kNfThreads / 64;
    const uint64_t step = (uint64_t)gridDim.x * kWaves * kNfUnroll;
    uint32_t cur = 0;   // the tensor of the wave's last word
    // workgroup-iteration i covers bitmap words [i*16, i*16+16): wave v takes
    // words 4k + v, k < kNfUnroll, one group per lane
    for (uint64_t base = (uint64_t)blockIdx.x * kWaves * kNfUnroll; base < a.n_words; base += step) {
        v3u slot[kNfUnroll];
        uint64_t flags[kNfUnroll];
        uint32_t prefix[kNfUnroll], tens[kNfUnroll];
        uint64_t group[kNfUnroll];
#pragma unroll
        for (int k = 0; k < kNfUnroll; ++k) {
            const uint64_t w = base + kWaves * k + wave;
            tens[k] = 0;
            group[k] = ~uint64_t(0);
            if (w < a.n_words) {
                advance_to(a, w, cur);
                const uint32_t t = cur;
                const Nf12Tensor &T = a.t[t];
                const uint64_t wl = w - T.word_base;
                const uint64_t g = 64 * wl + lane;
                tens[k] = t;
                // (the wave's 64 groups share one bitmap word: scalar loads)
                flags[k] = *(const __attribute__((address_space(4))) uint64_t *)(T.flags + wl);
                prefix[k] = *(const __attribute__((address_space(4))) uint32_t *)(T.prefix + wl);
                if (g < T.n_groups) {
                    group[k] = g;
                    slot[k] = __builtin_nontemporal_load(reinterpret_cast<const v3u *>(T.slots + 12 * g));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kNfUnroll; ++k) {
            const uint64_t g = group[k];
            if (g == ~uint64_t(0)) continue;
            const Nf12Tensor &T = a.t[tens[k]];
            v4u v = expand(slot[k]);
            if (((flags[k] >> lane) & 1u) && T.n_escaped) {
                // the escape entry of this outlier, kept inside the buffer
                // whatever the device bytes say
                uint64_t r = prefix[k] + (uint64_t)__builtin_popcountll(flags[k] & below);
                r = r < T.n_escaped ? r : T.n_escaped - 1;
                v = *reinterpret_cast<const v4u *>(T.escape + 16 * r);
            }
            const uint64_t j = 8 * g;
            if (j + 8 <= T.n) {
                __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(T.out + j));
            } else {
                for (uint32_t i = 0; j + i < T.n; ++i) {
                    const uint32_t wd = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
                    T.out[j + i] = (uint16_t)(wd >> (16 * (i & 1u)));
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_nf12_decode(const Nf12Args &args, int max_grid, hipStream_t stream) {
    const uint64_t per_wg = (uint64_t)(kNfThreads / 64) * kNfUnroll;   // bitmap words per step
    const uint64_t need = (args.n_words + per_wg - 1) / per_wg;
    const int grid = (int)(need < (uint64_t)max_grid ? need : (uint64_t)max_grid);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(nf12_decode_kernel, dim3(grid), dim3(kNfThreads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace df11
