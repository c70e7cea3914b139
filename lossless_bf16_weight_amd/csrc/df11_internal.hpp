// Internal layout shared by the host library and the HIP kernels.
#pragma once
#include <stdint.h>

#include "../../include/df11.h"

namespace df11 {

// Container version 4 constants (layout documented in include/df11.h).
constexpr uint32_t kVersion = 4;
constexpr uint32_t kHeader = DF11_HEADER_BYTES;
constexpr uint32_t kChunk = DF11_CHUNK_ELEMS;
constexpr int kWindows = DF11_WINDOWS;
constexpr int kMaxLen = DF11_MAX_CODE_LEN;
// A window's 16-bit index entry: the number of codes that start in it (at
// most 1536: a window has at most ceil(24 * kChunk / kWindows) bits) in the
// low 11 bits, the offset of the first of them from the window's first bit
// (under 24) in the top 5; 0 for a window with no code start.
constexpr unsigned kWinGapShift = 11;
constexpr unsigned kWinCntMask = (1u << kWinGapShift) - 1u;
static_assert((24u * kChunk + kWindows - 1) / kWindows <= kWinCntMask, "window counts fit 11 bits");

// Exponent bytes are handled rotated right by one bit inside the decoder,
// rot(e) = (e >> 1) | (e & 1) << 7, so that a BF16 word splits into the two
// bytes [sign | e >> 1] and [e & 1 | fraction]: the decode tables hold rot(e)
// and the join of tile bytes with raw bytes is two bitfield inserts and two
// byte permutes per four words.
#if defined(__HIPCC__)
#define DF11_HD __host__ __device__
#else
#define DF11_HD
#endif
DF11_HD constexpr uint8_t rot_exp(unsigned e) {
    return (uint8_t)(((e >> 1) | (e << 7)) & 0xFFu);
}

// First bit of window i (0 <= i <= kWindows) of a chunk of nbits bits,
// counted from the chunk's first bit: the windows split the chunk's bits as
// evenly as integers allow.  (nbits <= 24 * kChunk, so i * nbits < 2^32.)
DF11_HD constexpr uint32_t window_edge(uint32_t nbits, uint32_t i) {
    return (i * nbits) / (uint32_t)kWindows;
}

// First-level decode table: indexed by the next kL1Bits bits of the stream,
// the first of them the lowest index bit.
// Entry: bits 0..23 up to three rotated exponent bytes (first code in the
// low byte), bits 24..28 how many stream bits they use, bits 29..30 how many
// codes (1..3).  An entry with count 0 names the second-level subtable of a
// prefix whose first code is longer than kL1Bits (or that no valid stream
// holds): F << 16 | (k + 1), below.
constexpr int kL1Bits = 10;
constexpr int kL1Size = 1 << kL1Bits;
constexpr int kMaxPerLookup = 3;
constexpr uint32_t kEntLenShift = 24;
constexpr uint32_t kEntCountShift = 29;
// Second level: one subtable per such prefix, indexed by its next k stream
// bits (first bit lowest), k = min(longest code under the prefix, kL2Bits) -
// kL1Bits, in canonical order from entry 2 on; entry rot(e) | (len | 1 << 5)
// << 8 (its high byte moved to bits 24..31 gives a one-code first-level
// entry), 0 for a code longer than kL2Bits (the canonical limits take it).
// Entries 0 and 1 stay 0: the subtable of the prefixes no valid stream holds
// and of those left over when the table is full.  F = 2 + (the subtable's
// byte offset) - (the prefix's last stream bit).
constexpr int kL2Bits = 16;
constexpr int kL2Max = 512;

// Per-tensor table record in device memory (and copied whole into LDS).
struct alignas(16) LutRecord {
    uint32_t l1[kL1Size];
    uint16_t l2[kL2Max];
    // lim[l]: 24-bit left-aligned exclusive upper bound of the codes of
    // length <= l (l = 1..24); a peeked 24-bit value v has a code of length l
    // exactly when lim[l-1] <= v < lim[l].
    uint32_t lim[32];
    // base[l] = (index of the first length-l symbol in `sorted`) - (its code)
    int32_t base[32];
    // rotated exponent bytes sorted by (code length, exponent)
    uint8_t sorted[256];
    // code length by rotated exponent byte (0 = absent)
    uint8_t len[256];
    uint32_t pad[4];
};
static_assert(sizeof(LutRecord) == 5904, "LUT record size");

// Builds a tensor's decode tables from its code lengths (host.cpp).
void build_lut(const uint8_t *len, LutRecord &R);

// Staged code bytes per chunk: chunks whose codes (plus 127 bits of slack,
// rounded out to 16 bytes) fit go through LDS, the others are read from
// global memory by the decode loop.
constexpr uint32_t kCodeCap = 13 * 1024;

// One chunk of one tensor, with everything the kernel needs to find its
// bytes, computed by the plan from the validated chunk index (the kernel
// never reads a container's chunk index).  Offsets are relative to the
// container's first byte.
struct alignas(16) ChunkRec {
    uint64_t stream_off;   // first staged stream byte (16-byte aligned)
    uint64_t raw_off;      // raw byte of the chunk's first element
    uint64_t win_off;      // the chunk's 512 window entries
    uint64_t reserved;
    uint32_t rel0;         // chunk's first stream bit - 8 * staged first byte
    uint32_t nbits;        // the chunk's stream bits
    uint32_t s_len;        // staged bytes (<= kCodeCap), bit 31: codes staged in LDS
    uint32_t nc;           // elements
    uint32_t raw_left;     // raw bytes from the chunk's first element (<= 64 KiB)
    uint32_t n_words;      // stream words from the staged first byte on (<= 2^25)
    uint32_t tensor;       // plan tensor index (decode tables)
    uint32_t chunk;        // chunk index within the tensor
};
static_assert(sizeof(ChunkRec) == 64, "chunk record size");
constexpr uint32_t kStagedBit = 0x80000000u;

// Work tickets.  A launch's workgroups take its chunks in order from a
// ticket counter: work[0] = tickets handed out past the first gridDim.x,
// work[1] = workgroups finished; the last workgroup to finish puts both back
// to zero and then writes the launch's id to the slot's completion word in
// host memory.  A plan holds kWorkSlots counters, 64 bytes apart; the host
// gives a launch only a slot whose previous launch has written its id (so no
// two running launches share a counter), and keeps for good the slot of a
// launch made while its stream is being captured (every replay of the graph
// uses it).
constexpr uint32_t kWorkSlots = 256;
constexpr uint32_t kWorkStride = 16;   // uint32 per counter slot
// Slots a plan lets captured launches hold.
constexpr uint32_t kGraphSlotsMax = kWorkSlots / 2;

// The host side of the slots.  issued[s]: id of the last launch given slot s
// (0: none yet); graph[s]: held by a captured launch.  fin[s] (host memory
// the device writes): id of the last launch on slot s that finished.
struct SlotTable {
    uint32_t seq = 0, next = 0, n_graph = 0;
    uint32_t issued[kWorkSlots] = {};
    bool graph[kWorkSlots] = {};
    // A free slot and the new launch's id (*id), or -1 when every slot is
    // held by a running launch or a captured one.
    int acquire(const uint32_t *fin, bool capture, uint32_t *id) {
        if (capture && n_graph >= kGraphSlotsMax) return -1;
        for (uint32_t i = 0; i < kWorkSlots; ++i) {
            const uint32_t s = (next + i) % kWorkSlots;
            if (graph[s]) continue;
            if (issued[s] != 0 && __atomic_load_n(&fin[s], __ATOMIC_ACQUIRE) != issued[s]) continue;
            if (++seq == 0) ++seq;
            issued[s] = seq;
            graph[s] = capture;
            n_graph += capture;
            next = s + 1;
            *id = seq;
            return (int)s;
        }
        return -1;
    }
    // A slot whose launch was never enqueued (the launch call failed).
    void release(int s) {
        if (graph[s]) --n_graph;
        graph[s] = false;
        issued[s] = 0;
    }
};

struct DecodeArgs {
    const ChunkRec *recs;        // the launch's chunks, in order
    const LutRecord *luts;       // plan's table records (indexed by plan tensor)
    uint32_t *status;            // plan's corruption flag
    uint32_t *work;              // this launch's ticket counter slot
    uint32_t *fin;               // the slot's completion word (host memory)
    uint32_t launch_id;          // written to *fin when the launch is done
    uint32_t n_items;
    uint32_t tensor_base;        // plan index of the launch's tensor 0
    const uint8_t *containers[DF11_MAX_BATCH];
    uint16_t *outs[DF11_MAX_BATCH];
};

// Encoder pieces shared by the host and the GPU encoders (encode.cpp): the
// length-limited canonical code of a histogram, the container layout for a
// total bit count, and the 512-byte header.
struct EncodeLayout {
    uint64_t n_chunks, total_bits;
    uint64_t off_ci, off_win, off_stream, stream_bytes, off_raw, raw_bytes, total;
};
void build_code(const uint64_t *freq, uint8_t *len, uint32_t *code);
EncodeLayout encode_layout(uint64_t n, uint64_t total_bits);
void write_header(uint8_t *out, uint64_t n, int ndim, const uint64_t *dims, const EncodeLayout &L,
                  const uint8_t *len);

// SHA-256 (FIPS 180-4) of `bytes` bytes (sha256.cpp).
void sha256(const void *data, uint64_t bytes, uint8_t out[32]);

// Records the error text that df11_last_error returns and gives back st
// (host.cpp; printf-style message).
df11_status report_error(df11_status st, const char *fmt, ...);

// Launches the decode kernel (decode.hip).  grid = number of workgroups.
hipError_t launch_decode(const DecodeArgs &args, int grid, hipStream_t stream);

// Workgroups of the decode kernel that fit on one compute unit at once.
int decode_wgs_per_cu();

// Launches the bandwidth-control kernel (control.hip): reads src_bytes, writes
// dst_bytes (both multiples of 16, pointers 16-byte aligned).
hipError_t launch_bw_control(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes,
                             int grid, hipStream_t stream);

}  // namespace df11
