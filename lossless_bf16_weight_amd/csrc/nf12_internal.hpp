// Internal layout of the NF12 format shared by its host code (nf12.cpp) and
// its kernel (nf12.hip).
#pragma once
#include "df11_internal.hpp"

namespace df11 {

// ---- NF12: the fixed-rate 12-bit format (layout in include/df11.h) -------

constexpr uint32_t kNf12Header = 256;
constexpr uint32_t kNf12Version = 1;
constexpr uint16_t kNf12PadWord = 0x3800;   // completes a partial last group; fits

struct Nf12Layout {
    uint64_t n, n_groups, n_words, n_escaped;
    uint64_t off_slots, off_flags, off_prefix, off_escape, total;
};

inline Nf12Layout nf12_layout(uint64_t n, uint64_t n_escaped) {
    auto up = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    Nf12Layout L;
    L.n = n;
    L.n_groups = (n + 7) / 8;
    L.n_words = (L.n_groups + 63) / 64;
    L.n_escaped = n_escaped;
    L.off_slots = kNf12Header;
    L.off_flags = up(L.off_slots + 12 * L.n_groups);
    L.off_prefix = up(L.off_flags + 8 * L.n_words);
    L.off_escape = up(L.off_prefix + 4 * L.n_words);
    L.total = up(L.off_escape + 16 * n_escaped);
    return L;
}

// One tensor of an NF12 launch.
struct Nf12Tensor {
    const uint8_t *slots;      // n_groups x 12 bytes
    const uint64_t *flags;     // outlier bitmaps, 64 groups per word
    const uint32_t *prefix;    // outlier counts before each bitmap word
    const uint8_t *escape;     // n_escaped x 16 bytes
    uint16_t *out;             // n words
    uint64_t n, n_groups, n_escaped;
    uint64_t word_base;        // the launch's bitmap words before this tensor's
};

// Tensors per NF12 launch (the kernel arguments hold their descriptors).
constexpr int kNf12MaxBatch = 24;

struct Nf12Args {
    Nf12Tensor t[kNf12MaxBatch];
    uint32_t n_tensors;
    uint64_t n_words;          // bitmap words (64-group units) over all tensors
};

// Launches the NF12 decode kernel (nf12.hip) with at most max_grid
// workgroups (nothing when there are no groups).
hipError_t launch_nf12_decode(const Nf12Args &args, int max_grid, hipStream_t stream);

}  // namespace df11
