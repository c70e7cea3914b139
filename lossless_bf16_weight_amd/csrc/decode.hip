// DFloat11-style decode kernel for gfx950 (CDNA4).
//
// Method (mlx-dfloat project page, introduction and 16-bit weight diagram):
// each BF16 weight is rebuilt from its raw byte (sign << 7 | 7-bit fraction)
// and its exponent byte, which is stored as a variable-length prefix code in
// one bitstream; output words are bit-identical to the originals.
//
// One workgroup = four wave64s (256 lanes) decodes whole chunks of 32768
// elements (64 KiB of BF16 output), one after the other; a launch's
// workgroups take its chunks from a ticket counter as they finish decoding
// the previous one.  A chunk takes two workgroup barriers: one before its
// decode, one after.  Per chunk:
//
//   1. index: the chunk's N bits form 512 windows (window i starts
//      floor(i*N/512) bits in); lane i takes windows 2i and 2i+1.  A DPP
//      prefix sum over each wave's lane totals of the window code counts,
//      plus the totals of the waves below (through LDS, written at the end
//      of the previous chunk's assembly), gives each window the chunk
//      position of its first code;
//   2. decode: each lane walks its two windows side by side (two
//      independent dependency chains; 512 chains per workgroup).  A chain
//      keeps the two code words around its position in registers; a
//      look-up funnel-shifts them, reads one first-level table entry (up to
//      three codes of <= 10 bits; codes of 11..16 bits use a subtable the
//      entry names, longer ones the canonical limits) together with the next
//      code word, and ORs the exponent bytes (rotated, see rot_exp) into a
//      32 KiB LDS tile, zero beforehand, at their chunk positions.  A counted
//      loop with no per-lane control flow runs while no window of the wave
//      can run out before its last counted look-up (each look-up takes at
//      most three codes) and no peek can pass the end of the staged words
//      (each moves a window at most 24 bits); a masked loop finishes;
//   3. check: a window must end exactly where the next non-empty window's
//      first code starts (or at the chunk end); otherwise the plan's flag is
//      set;
//   4. assemble: per 2048 elements, each lane joins 8 tile bytes with 8 raw
//      bytes into BF16 words (two bitfield inserts and two byte permutes per
//      four words), writes them with one 16-byte store, contiguous across the
//      wave (1 KiB per store instruction), and clears the tile bytes it read;
//      the next chunk's window entries, code bytes, tables and raw bytes are
//      requested meanwhile;
//   5. stage: at the end of its assembly each wave puts the next chunk's
//      code bytes in LDS as 32-bit words with the stream's first bit lowest,
//      writes its tables, and scans its windows (step 1 for the next chunk).
//      The raw bytes wait in registers (8 bytes per lane per 2048 elements)
//      until that chunk's assembly.
//
// There is no matrix arithmetic here: the path is bound by HBM traffic
// (about 1.36 bytes read and 2 bytes written per element), with the look-up
// chains' latency and integer ALU as the secondary limit.
#include <hip/hip_runtime.h>

#include "df11_internal.hpp"

namespace df11 {

constexpr int kThreads = 256;                      // lanes per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kTileBytes = kChunk;                 // one exponent byte per element
constexpr uint32_t kTilePadded = kTileBytes + kTileBytes / 32;   // 4 pad bytes per 128
// LDS per workgroup: 13 KiB staged codes + 33 KiB tile + 5.8 KiB tables +
// tickets and wave totals = 52 KiB, so that three workgroups
// fit in a compute unit's 160 KiB.
constexpr int kCodeWords = kCodeCap / 4;
constexpr int kCodeLoads = (kCodeCap + 16 * kThreads - 1) / (16 * kThreads);
constexpr int kBlockElems = 8 * kThreads;          // elements per store block
constexpr int kBlocks = kChunk / kBlockElems;
static_assert(kBlockElems == 2048 && kThreads == 256, "block tile stride 2112");
static_assert(2 * kThreads == kWindows, "two windows per lane");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Global memory, named as such: loads and stores through these pointers are
// global instructions, never flat ones (a flat store also counts against the
// LDS wait counter, so every LDS wait after it would wait for the store too),
// whatever the compiler can infer about where a pointer points.
#define GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ GLOBAL T *global(T *p) {
    return (GLOBAL T *)p;
}

// A pointer that is the same for all lanes, made a scalar value, so that an
// access through it plus a lane offset uses the scalar base + vector offset
// address form (no 64-bit vector address per access).
template <class T>
__device__ __forceinline__ GLOBAL T *uniform(GLOBAL T *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (GLOBAL T *)((uint64_t)hi << 32 | lo);
}

// LDS of one workgroup.  Staged code word k (first stream bit lowest) sits
// in codes[k + 1], with codes[1] 16-byte aligned; the 12 bytes in front keep
// codes[0] inside the struct.  The tile's and the tables' bases fold into
// the instructions' 16-bit offsets.
struct Lds {
    uint32_t pad[3];
    uint32_t codes[kCodeWords + 9];   // 12 + 4 * (kCodeWords + 9) = 0 mod 16
    uint8_t tile[kTilePadded + 16];
    LutRecord lut;
    // the next work item's ticket (slot = iteration parity), written by wave
    // 0 before the barrier that ends the decode (n_items or more: no item)
    uint32_t rec_id[2];
    // per wave: bit offset from the chunk start of the first code of its
    // first non-empty window (~0: all its windows are empty), and the number
    // of codes its windows hold
    uint32_t wave_first[2][kWaves];
    uint32_t wave_total[2][kWaves];
};
static_assert(offsetof(Lds, tile) % 16 == 0 && offsetof(Lds, lut) % 16 == 0,
              "LDS alignment");
static_assert(sizeof(Lds) <= 53248, "three workgroups per compute unit");

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

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = min(x, (uint32_t)__shfl_xor((int)x, m));
    return x;
}

// Four BF16 words from four rotated exponent bytes t and four raw bytes r:
// the high bytes (sign | e >> 1) and the low bytes (e & 1 | fraction) of all
// four with one bitfield insert each, then interleaved by two byte permutes.
__device__ __forceinline__ u32x2 join4(uint32_t t, uint32_t r) {
    const uint32_t hi = (r & 0x80808080u) | (t & 0x7F7F7F7Fu);
    const uint32_t lo = (t & 0x80808080u) | (r & 0x7F7F7F7Fu);
    return u32x2{__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u)};
}

__device__ __forceinline__ u32x4 join8(u32x2 t8, u32x2 r8) {
    const u32x2 a = join4(t8.x, r8.x), b = join4(t8.y, r8.y);
    return u32x4{a.x, a.y, b.x, b.y};
}

// ---- code sources ---------------------------------------------------------
// Source words hold the stream least significant bit first: bit i of word k
// is stream bit 32 (k - 1) + i (the stream itself is most significant bit
// first within each byte, so a stored word is byte-swapped and bit-reversed
// on its way in).  A window's position is kept as P = p + 30, p its stream
// bit offset from the source's first word: the funnel shift of words k+1:k
// with k = P / 32 by P mod 32 then yields the stream bits from p - 2 on, so
// that bits 2..11 are the next 10 stream bits -- already the byte offset of
// their first-level table entry (the table is indexed by those bits in
// stream order, first bit lowest).

__device__ __forceinline__ uint32_t lsb_first(uint32_t stored) {
    return __builtin_bitreverse32(bswap32(stored));
}

constexpr uint32_t kPosBias = 30;

struct LdsCodes {
    static constexpr bool kLds = true;
    const uint32_t *w;   // w[k] = staged word k-1, least significant bit first
    uint32_t pmax;       // largest P whose words are inside
};

struct GlobalCodes {
    static constexpr bool kLds = false;
    const GLOBAL uint32_t *w;   // w[k] = stream word k-1, as stored
    uint32_t pmax;
    __device__ __forceinline__ uint32_t peek(uint32_t P) const {
        const uint32_t k = P >> 5;
        return __builtin_amdgcn_alignbit(lsb_first(w[k + 1]), lsb_first(w[k]), P);
    }
};

// First-level style entry of one code of `len` bits and rotated exponent
// byte `sym`.
__device__ __forceinline__ uint32_t one_code(uint32_t sym, uint32_t len) {
    return sym | (len << kEntLenShift) | (1u << kEntCountShift);
}

// A first-level entry that names a second-level subtable (its count is 0).
__device__ __forceinline__ bool is_long(uint32_t ent) { return ent < (1u << kEntCountShift); }

// Entry for a code longer than kL2Bits from the canonical limits; msb = the
// next 30 stream bits, first bit highest.  A prefix no valid stream holds
// sets `bad` and yields a 24-bit code of exponent 0.
__device__ __forceinline__ uint32_t limits_entry(const LutRecord &T, uint32_t msb, uint32_t &bad) {
    const uint32_t v = msb >> (32 - kMaxLen);
    uint32_t l = kL1Bits + 1;
    while (l <= (uint32_t)kMaxLen && v >= T.lim[l]) ++l;
    if (l > (uint32_t)kMaxLen) {
        bad = 1;
        return one_code(0u, kMaxLen);
    }
    return one_code(T.sorted[(int)(v >> (kMaxLen - l)) + T.base[l]], l);
}

// Entries for codes longer than kL1Bits, for both chains at once (ea / eb
// are replaced where they name a subtable; ta / tb are the peeked words,
// the code from bit 2 on).  The subtable entry's byte address is
// l2 - 2 + F + bfe(peek, 11, k + 1) with F << 16 | (k + 1) the first-level
// entry: the k + 1 bits from the prefix's last bit on are twice the index
// plus that bit, which F takes off again.  Both chains' reads go out
// together, one LDS round trip for the pair, and the u16 entry becomes a
// first-level entry with one byte permute.  A code longer than kL2Bits then
// takes the canonical limits.
__device__ __forceinline__ void long_pair(const LutRecord &T, uint32_t ta, uint32_t tb, uint32_t &ea, uint32_t &eb,
                                          uint32_t &bad) {
    const bool la = is_long(ea), lb = is_long(eb);
    const uint8_t *l2 = reinterpret_cast<const uint8_t *>(T.l2) - 2;
    // (a chain with a short code reads entry 0, so that both reads are
    // unconditional and inside the table)
    const uint32_t ia = la ? (ea >> 16) + __builtin_amdgcn_ubfe(ta, 11, ea) : 2u;
    const uint32_t ib = lb ? (eb >> 16) + __builtin_amdgcn_ubfe(tb, 11, eb) : 2u;
    const uint32_t ra = *reinterpret_cast<const uint16_t *>(l2 + ia);
    const uint32_t rb = *reinterpret_cast<const uint16_t *>(l2 + ib);
    // byte 0 stays, byte 1 (length | 1 << 5) moves to byte 3
    ea = la ? __builtin_amdgcn_perm(0u, ra, 0x010C0C00u) : ea;
    eb = lb ? __builtin_amdgcn_perm(0u, rb, 0x010C0C00u) : eb;
    if (__builtin_expect((la && ra == 0) | (lb && rb == 0), 0)) {
        if (la && ra == 0) ea = limits_entry(T, __builtin_bitreverse32(ta >> 2), bad);
        if (lb && rb == 0) eb = limits_entry(T, __builtin_bitreverse32(tb >> 2), bad);
    }
}

__device__ __forceinline__ uint32_t ent_count(uint32_t ent) { return ent >> kEntCountShift; }
__device__ __forceinline__ uint32_t ent_bits(uint32_t ent) { return (ent >> kEntLenShift) & 31u; }

// Both chains' look-up entries with the code words read from the stream in
// global memory (chunks whose codes are not staged in LDS).  kClamp: clamp
// the positions to the source.
template <bool kClamp>
__device__ __forceinline__ void entries(const Lds &L, const GlobalCodes &src, uint32_t pa,
                                        uint32_t pb, uint32_t &ea, uint32_t &eb, uint32_t &bad) {
    if (kClamp) {
        pa = min(pa, src.pmax);
        pb = min(pb, src.pmax);
    }
    const uint8_t *l1 = reinterpret_cast<const uint8_t *>(L.lut.l1);
    const uint32_t ta = src.peek(pa);
    const uint32_t tb = src.peek(pb);
    ea = *reinterpret_cast<const uint32_t *>(l1 + (ta & ((kL1Size - 1) << 2)));
    eb = *reinterpret_cast<const uint32_t *>(l1 + (tb & ((kL1Size - 1) << 2)));
    if (__builtin_expect(is_long(ea) | is_long(eb), 0)) long_pair(L.lut, ta, tb, ea, eb, bad);
}

// One window's decoder.  The tile is cleared before the decode, and every
// look-up ORs its exponent bytes into the tile dword at the chain's next
// output position; the bytes that run past that dword are ORed in by the
// chain's next look-up, together with its own (one LDS OR per look-up
// instead of two, 1.5% faster), and the last ones after the window's loop.
// So chains never overwrite each other's bytes: where a window's last
// look-up decodes codes of the next window (its last entry can run up to two
// codes past the window's end), it ORs in the same values that the next
// window's chain writes there.
struct Chain {
    uint32_t P;      // stream position of the next code, plus kPosBias
    uint32_t p8;     // 8 x the next output position (chunk-relative)
    uint32_t qe;     // the window's end (output position)
    uint32_t spill;  // bytes of the last look-up past its dword, for the next dword
};

// Byte offset in the tile of dword dw: 4 pad bytes after every 128, so that
// the dwords lanes store at the same time (their windows' outputs start
// about 64 positions apart) spread over the banks.  The pads stay zero.
__device__ __forceinline__ uint32_t tile_off(uint32_t dw) { return (dw + (dw >> 5)) << 2; }

__device__ __forceinline__ void tile_or(Lds &L, uint32_t off, uint32_t v) {
    uint32_t *d = static_cast<uint32_t *>(__builtin_assume_aligned(L.tile + off, 4));   // off % 4 == 0
    __hip_atomic_fetch_or(d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Chain c takes look-up entry ent (0 for a finished chain in the masked
// phase: it then ORs zeros and keeps its state).
__device__ __forceinline__ void step(Lds &L, Chain &c, uint32_t ent) {
    // the entry's bytes from the position's byte in its dword on, with the
    // previous look-up's spill (whose dword this is); the bytes past the
    // dword wait for the next look-up, whose dword they are in
    const uint64_t x = (uint64_t)(ent & 0xFFFFFFu) << (c.p8 & 24u);
    const uint32_t off = tile_off(c.p8 >> 5);
    tile_or(L, off, (uint32_t)x | c.spill);
    c.spill = (uint32_t)(x >> 32);
    // p8 += 8 x count as one v_lshl_add (the compiler's shift, mask and add
    // is one VALU instruction more per chain and look-up)
    uint32_t p8;
    asm("v_lshl_add_u32 %0, %1, 3, %2" : "=v"(p8) : "v"(ent_count(ent)), "v"(c.p8));
    c.p8 = p8;
    c.P += ent_bits(ent);
}

__device__ __forceinline__ uint32_t out_pos(const Chain &c) { return c.p8 >> 3; }

// The masked phase for a source in global memory (see masked_window_tail).
__device__ __forceinline__ void masked_tail(Lds &L, const GlobalCodes &src, Chain &A, Chain &B, int32_t &ra,
                                            int32_t &rb, uint32_t &ea_r, uint32_t &eb_r, uint32_t &bad) {
    uint32_t ea, eb;
    bool any = __ballot((ra > 0) | (rb > 0)) != 0;
    while (any) {
        const bool aa = ra > 0, ab = rb > 0;
        entries<true>(L, src, A.P, B.P, ea, eb, bad);
        ea = aa ? ea : 0u;
        eb = ab ? eb : 0u;
        ea_r = aa ? ea : ea_r;
        eb_r = ab ? eb : eb_r;
        ra -= (int32_t)ent_count(ea);
        rb -= (int32_t)ent_count(eb);
        step(L, A, ea);
        step(L, B, eb);
        any = __ballot((ra > 0) | (rb > 0)) != 0;
    }
}

// Bits taken by the last k codes of an entry (k < its count).
__device__ __forceinline__ uint32_t trailing_bits(const Lds &L, uint32_t ent, uint32_t k) {
    uint32_t c = 0;
    const uint32_t n = ent_count(ent);
    for (uint32_t j = n - k; j < n; ++j) c += L.lut.len[(ent >> (8 * j)) & 0xFFu];
    return c;
}

// The code words a chain's peeks read, in registers: w0, w1 = staged words
// k, k+1 with k = P / 32.  Each look-up also reads word k+2, with its table
// entry, and shifts it in when the look-up moves the chain into the next
// word; so a look-up waits on one LDS round trip (the table entry and that
// word together) instead of two in a row.
struct Window {
    uint32_t w0, w1;
    uint32_t kb;   // 4 (P / 32): byte offset of word k from codes[0]
};

__device__ __forceinline__ Window window_at(const uint32_t *w, uint32_t P) {
    const uint32_t k = P >> 5;
    return Window{w[k], w[k + 1], (P >> 3) & ~3u};
}

// The long-code path for one chain (see long_pair).
__device__ __forceinline__ void long_one(const LutRecord &T, uint32_t t, uint32_t &e, uint32_t &bad) {
    const bool l = is_long(e);
    const uint8_t *l2 = reinterpret_cast<const uint8_t *>(T.l2) - 2;
    const uint32_t i = l ? (e >> 16) + __builtin_amdgcn_ubfe(t, 11, e) : 2u;
    const uint32_t r = *reinterpret_cast<const uint16_t *>(l2 + i);
    e = l ? __builtin_amdgcn_perm(0u, r, 0x010C0C00u) : e;
    if (__builtin_expect(l && r == 0, 0)) e = limits_entry(T, __builtin_bitreverse32(t >> 2), bad);
}

// One look-up of one chain whose table entry e and next word n were read
// half an iteration earlier; then the reads for its next look-up go out, so
// that they are in flight while the other chain's look-up computes.
__device__ __forceinline__ void half_step(Lds &L, Chain &c, Window &w, uint32_t &t, uint32_t &e, uint32_t &n,
                                          uint32_t &e_last, uint32_t &bad) {
    const uint8_t *l1 = reinterpret_cast<const uint8_t *>(L.lut.l1);
    const uint8_t *cw = reinterpret_cast<const uint8_t *>(L.codes);
    uint32_t ent = e;
    if (__builtin_expect(is_long(ent), 0)) long_one(L.lut, t, ent, bad);
    const uint32_t kn = ((c.P + ent_bits(ent)) >> 3) & ~3u;
    const bool cr = kn != w.kb;
    w.kb = kn;
    w.w0 = cr ? w.w1 : w.w0;
    w.w1 = cr ? n : w.w1;
    step(L, c, ent);
    e_last = ent;
    t = __builtin_amdgcn_alignbit(w.w1, w.w0, c.P);
    e = *reinterpret_cast<const uint32_t *>(l1 + (t & ((kL1Size - 1) << 2)));
    n = *reinterpret_cast<const uint32_t *>(cw + w.kb + 8);
}

// T counted look-ups of both chains, software-pipelined by half an
// iteration: each chain's table entry and next word are read while the
// other chain's look-up computes, so that a wave hides part of its own LDS
// round trips (2% faster at 20/5 than both chains in lock step, 0.7% in
// steady state).  Two iterations per loop turn, so that the loop-carried
// registers need no copies.
__device__ __forceinline__ void pipelined_steps(Lds &L, Chain &A, Chain &B, Window &wa, Window &wb, uint32_t T,
                                                uint32_t &bad, uint32_t &ea_o, uint32_t &eb_o) {
    if (T == 0) return;
    const uint8_t *l1 = reinterpret_cast<const uint8_t *>(L.lut.l1);
    const uint8_t *cw = reinterpret_cast<const uint8_t *>(L.codes);
    uint32_t ta = __builtin_amdgcn_alignbit(wa.w1, wa.w0, A.P);
    uint32_t ea = *reinterpret_cast<const uint32_t *>(l1 + (ta & ((kL1Size - 1) << 2)));
    uint32_t na = *reinterpret_cast<const uint32_t *>(cw + wa.kb + 8);
    uint32_t tb = __builtin_amdgcn_alignbit(wb.w1, wb.w0, B.P);
    uint32_t eb = *reinterpret_cast<const uint32_t *>(l1 + (tb & ((kL1Size - 1) << 2)));
    uint32_t nb = *reinterpret_cast<const uint32_t *>(cw + wb.kb + 8);
    uint32_t i = 0;
    for (; i + 1 < T; i += 2) {
        half_step(L, A, wa, ta, ea, na, ea_o, bad);
        half_step(L, B, wb, tb, eb, nb, eb_o, bad);
        half_step(L, A, wa, ta, ea, na, ea_o, bad);
        half_step(L, B, wb, tb, eb, nb, eb_o, bad);
    }
    if (i < T) {
        half_step(L, A, wa, ta, ea, na, ea_o, bad);
        half_step(L, B, wb, tb, eb, nb, eb_o, bad);
    }
}

// One look-up of both chains in the masked phase, from register windows:
// as half_step, in lock step, for the chains whose windows still have codes
// (aa / ab; the others take a zero entry and keep their state).  The
// next-word reads are clamped to the staged words, so a container whose
// index disagrees with its stream reads inside them.  aa / ab come back for
// the next look-up.  (Pipelining this phase as well measured no faster.)
__device__ __forceinline__ void masked_window_step(Lds &L, uint32_t kmax4, Chain &A, Chain &B, Window &wa,
                                                   Window &wb, int32_t &ra, int32_t &rb, uint32_t &ea_r,
                                                   uint32_t &eb_r, uint32_t &bad, bool &aa, bool &ab) {
    const uint8_t *l1 = reinterpret_cast<const uint8_t *>(L.lut.l1);
    const uint8_t *cw = reinterpret_cast<const uint8_t *>(L.codes);
    const uint32_t ta = __builtin_amdgcn_alignbit(wa.w1, wa.w0, A.P);
    const uint32_t tb = __builtin_amdgcn_alignbit(wb.w1, wb.w0, B.P);
    uint32_t ea = *reinterpret_cast<const uint32_t *>(l1 + (ta & ((kL1Size - 1) << 2)));
    uint32_t eb = *reinterpret_cast<const uint32_t *>(l1 + (tb & ((kL1Size - 1) << 2)));
    const uint32_t na = *reinterpret_cast<const uint32_t *>(cw + min(wa.kb, kmax4) + 8);
    const uint32_t nb = *reinterpret_cast<const uint32_t *>(cw + min(wb.kb, kmax4) + 8);
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_expect(is_long(ea) | is_long(eb), 0)) long_pair(L.lut, ta, tb, ea, eb, bad);
    ea = aa ? ea : 0u;
    eb = ab ? eb : 0u;
    ea_r = aa ? ea : ea_r;
    eb_r = ab ? eb : eb_r;
    ra -= (int32_t)ent_count(ea);
    rb -= (int32_t)ent_count(eb);
    const uint32_t ka = ((A.P + ent_bits(ea)) >> 3) & ~3u;
    const uint32_t kb = ((B.P + ent_bits(eb)) >> 3) & ~3u;
    const bool ca = ka != wa.kb;
    const bool cb = kb != wb.kb;
    wa.kb = ka;
    wb.kb = kb;
    wa.w0 = ca ? wa.w1 : wa.w0;
    wa.w1 = ca ? na : wa.w1;
    wb.w0 = cb ? wb.w1 : wb.w0;
    wb.w1 = cb ? nb : wb.w1;
    step(L, A, ea);
    step(L, B, eb);
    aa = ra > 0;
    ab = rb > 0;
}

// The masked phase: look-ups while any window of the wave has codes left
// (two per loop iteration, so that the loop-carried registers need no
// copies).
__device__ __forceinline__ void masked_window_tail(Lds &L, uint32_t kmax4, Chain &A, Chain &B, Window &wa,
                                                   Window &wb, int32_t &ra, int32_t &rb, uint32_t &ea_r,
                                                   uint32_t &eb_r, uint32_t &bad) {
    bool aa = ra > 0, ab = rb > 0;
    if (__ballot(aa | ab) == 0) return;
    do {
        masked_window_step(L, kmax4, A, B, wa, wb, ra, rb, ea_r, eb_r, bad, aa, ab);
        if (__ballot(aa | ab) == 0) break;
        masked_window_step(L, kmax4, A, B, wa, wb, ra, rb, ea_r, eb_r, bad, aa, ab);
    } while (__ballot(aa | ab) != 0);
}

// Decode both windows of this lane.  T: look-ups before whose last one no
// window of the wave has run out of codes (codes in global memory: after
// whose last one).  On return A.P / B.P hold the stream positions (plus
// kPosBias) where the windows' last codes end.
template <class Src>
__device__ __forceinline__ void decode_pair(Lds &L, const Src &src, Chain &A, Chain &B, uint32_t T,
                                            uint32_t &bad) {
    uint32_t ea, eb;
    int32_t ra, rb;
    uint32_t ea_r = 0, eb_r = 0;
    // 1. counted (the caller keeps the starts at least 24*T bits below the
    //    source's end, so these peeks need no clamp); 2. masked, without
    //    branches: a finished window takes a zero entry; each window's last
    //    entry is kept to find where its last code ends
    if constexpr (Src::kLds) {
        Window wa = window_at(src.w, A.P), wb = window_at(src.w, B.P);
        // (the loop then starts with no LDS read in flight)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        pipelined_steps(L, A, B, wa, wb, T, bad, ea_r, eb_r);
        // (a window may have run out during the last counted look-up: its
        // last entry is then that look-up's)
        ra = (int32_t)(A.qe - out_pos(A));
        rb = (int32_t)(B.qe - out_pos(B));
        masked_window_tail(L, 4u * (src.pmax >> 5), A, B, wa, wb, ra, rb, ea_r, eb_r, bad);
    } else {
        for (uint32_t t = 0; t < T; ++t) {
            entries<false>(L, src, A.P, B.P, ea, eb, bad);
            step(L, A, ea);
            step(L, B, eb);
        }
        ra = (int32_t)(A.qe - out_pos(A));
        rb = (int32_t)(B.qe - out_pos(B));
        masked_tail(L, src, A, B, ra, rb, ea_r, eb_r, bad);
    }
    // the last spills
    tile_or(L, tile_off(A.p8 >> 5), A.spill);
    tile_or(L, tile_off(B.p8 >> 5), B.spill);
    // the last entry took -r codes past the window's end
    A.P -= trailing_bits(L, ea_r, (uint32_t)(-ra));
    B.P -= trailing_bits(L, eb_r, (uint32_t)(-rb));
}

// One work item (a chunk of a tensor) and where its bytes are.
struct Item {
    const GLOBAL uint8_t *stream;   // the staged stream bytes
    const GLOBAL uint8_t *raw;      // raw bytes from the chunk's first element
    const GLOBAL uint8_t *win;      // the chunk's window entries
    GLOBAL uint16_t *out;           // output from the chunk's first element
    uint32_t rel0, nbits;    // the chunk's stream bits, relative to the staged bytes
    uint32_t s_len;          // staged bytes
    uint32_t staged;         // the chunk's codes go through LDS
    uint32_t nc;             // elements
    uint32_t raw_left;       // raw bytes from the chunk's first element
    uint32_t n_words;        // stream words from the staged first byte on
    uint32_t lut;            // plan tensor index
};

// A chunk record (id is the same for all lanes): one scalar load of its 64
// bytes through the constant address space, so every field is in a scalar
// register and no workgroup barrier is needed to share it.
#define CONSTANT __attribute__((address_space(4)))
__device__ __forceinline__ Item item_at(const DecodeArgs &a, uint32_t id) {
    const CONSTANT ChunkRec *r = (const CONSTANT ChunkRec *)a.recs + id;
    const uint64_t stream_off = r->stream_off, raw_off = r->raw_off, win_off = r->win_off;
    const uint32_t tensor = r->tensor, chunk = r->chunk;
    const uint32_t tl = tensor - a.tensor_base;
    const GLOBAL uint8_t *C = global(a.containers[tl]);
    Item it;
    it.stream = C + stream_off;
    it.raw = C + raw_off;
    it.win = C + win_off;
    it.out = global(a.outs[tl]) + (uint64_t)chunk * kChunk;
    it.rel0 = r->rel0;
    it.nbits = r->nbits;
    const uint32_t sl = r->s_len;
    it.s_len = sl & ~kStagedBit;
    it.staged = sl >> 31;
    it.nc = r->nc;
    it.raw_left = r->raw_left;
    it.n_words = r->n_words;
    it.lut = tensor;
    return it;
}
static_assert(offsetof(ChunkRec, rel0) == 32 && offsetof(ChunkRec, tensor) == 56, "record layout");

// Wave 0: the next ticket of the launch (lane 0 takes it, every lane gets
// it).  Tickets count on from gridDim.x: workgroup w's first item is w.
__device__ __forceinline__ uint32_t take_ticket(const DecodeArgs &a, uint32_t lane) {
    uint32_t t = 0;
    if (lane == 0) t = atomicAdd(a.work, 1u);
    return gridDim.x + __builtin_amdgcn_readfirstlane(t);
}

// The decode tables of a tensor, 16 bytes per lane per 4 KiB.
constexpr int kLutLoads = (int)((sizeof(LutRecord) / 16 + kThreads - 1) / kThreads);
static_assert(sizeof(LutRecord) % 16 == 0, "table record size");
__device__ __forceinline__ void load_lut(const DecodeArgs &a, uint32_t lut, uint32_t tid, u32x4 (&lr)[kLutLoads]) {
    const GLOBAL u32x4 *src = reinterpret_cast<const GLOBAL u32x4 *>(global(a.luts) + lut);
#pragma unroll
    for (int k = 0; k < kLutLoads; ++k)
        lr[k] = src[min(kThreads * k + tid, (uint32_t)(sizeof(LutRecord) / 16 - 1))];
}
__device__ __forceinline__ void put_lut(Lds &L, uint32_t tid, const u32x4 (&lr)[kLutLoads]) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(&L.lut);
#pragma unroll
    for (int k = 0; k < kLutLoads; ++k)
        if (kThreads * k + tid < sizeof(LutRecord) / 16) dst[kThreads * k + tid] = lr[k];
}

// The staged code bytes of an item: 16 bytes per lane per 4 KiB.  Past the
// chunk's bytes the address repeats (a cache hit, no extra HBM traffic) so
// that the load count stays fixed.
__device__ __forceinline__ void load_codes(const Item &it, uint32_t tid, u32x4 (&cw)[kCodeLoads]) {
    const GLOBAL uint8_t *stream = it.stream;
#pragma unroll
    for (int k = 0; k < kCodeLoads; ++k) {
        const uint32_t off = min(16u * kThreads * k + 16u * tid, it.s_len - 16u);
        // (non-temporal: plain loads measured about 6% slower overall)
        cw[k] = __builtin_nontemporal_load(reinterpret_cast<const GLOBAL u32x4 *>(stream + off));
    }
}

// Raw bytes of store block b (elements 2048b + 8 tid .. +8) of an item; a
// partial chunk reads inside its (16-byte padded) raw bytes only.
__device__ __forceinline__ u32x2 load_raw(const Item &it, uint32_t tid, int b) {
    // a block base shared by the wave and a lane offset, both clamped for a
    // partial chunk to the last whole 8 bytes
    uint32_t base = kBlockElems * b, lim = ~0u;
    if (it.nc != (uint32_t)kChunk) {
        const uint32_t last = (it.raw_left - 8u) & ~7u;
        base = min(base, last);
        lim = last - base;
    }
    const GLOBAL uint8_t *rb = uniform(it.raw + base);
    // (a plain load: the non-temporal hint measured about 8% slower here)
    return *reinterpret_cast<const GLOBAL u32x2 *>(rb + min(8u * tid, lim));
}

// The index entries of this lane's windows 2 tid (low half) and 2 tid + 1
// (high half), each count | gap << kWinGapShift.  (Non-temporal, as the
// code bytes: about 1% faster here.)
__device__ __forceinline__ uint32_t load_windows(const Item &it, uint32_t tid) {
    return __builtin_nontemporal_load(reinterpret_cast<const GLOBAL uint32_t *>(it.win) + tid);
}

// The staged code bytes of an item to LDS, first stream bit lowest.
__device__ __forceinline__ void stage_codes(Lds &L, uint32_t tid, const u32x4 (&cw)[kCodeLoads]) {
#pragma unroll
    for (int q = 0; q < kCodeLoads; ++q) {
        if (16u * kThreads * q + 16u * tid < (uint32_t)kCodeCap) {
            u32x4 v = cw[q];
            v.x = lsb_first(v.x);
            v.y = lsb_first(v.y);
            v.z = lsb_first(v.z);
            v.w = lsb_first(v.w);
            reinterpret_cast<u32x4 *>(L.codes + 1)[kThreads * q + tid] = v;
        }
    }
}

// Windows 2 tid (a) and 2 tid + 1 (b) of an item: code counts, first code
// starts (bit offsets from the staged first byte) and the wave's inclusive
// count sum; the wave's total and first code go to LDS slot `slot` for the
// waves above it.
struct WinScan {
    uint32_t na, nb, sa, sb, incl, first;
    uint64_t mask;   // lanes with a code
};
__device__ __forceinline__ WinScan scan_windows(Lds &L, const Item &it, uint32_t win, uint32_t tid, uint32_t lane,
                                                uint32_t wave, uint32_t slot) {
    WinScan w;
    w.na = win & kWinCntMask;
    w.nb = (win >> 16) & kWinCntMask;
    w.incl = wave_inclusive_sum(w.na + w.nb);
    w.sa = it.rel0 + window_edge(it.nbits, 2 * tid) + ((win >> kWinGapShift) & 31u);
    w.sb = it.rel0 + window_edge(it.nbits, 2 * tid + 1) + (win >> (16 + kWinGapShift));
    w.mask = __ballot(w.na + w.nb != 0);
    w.first = w.na ? w.sa : w.sb;
    const uint32_t wf = __shfl(w.first, w.mask ? (int)__builtin_ctzll(w.mask) : 0);
    if (lane == 63) L.wave_total[slot][wave] = w.incl;
    if (lane == 0) L.wave_first[slot][wave] = w.mask ? wf : 0xFFFFFFFFu;
    return w;
}

__global__ __launch_bounds__(kThreads, 3) void decode_kernel(DecodeArgs a) {
    __shared__ Lds L;
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u, wave = tid >> 6;
    const uint32_t n = a.n_items;   // >= gridDim.x
    uint32_t bad_any = 0;

    // Software pipeline over the workgroup's items: while item i is
    // assembled, the code bytes, window entries and decode tables of item
    // i+1 are in flight, and its raw bytes are requested block by block as
    // item i's assembly frees the registers.  At the end of its assembly a
    // wave stages item i+1's code bytes, puts its tables in LDS and scans its
    // windows, and the assembly leaves the tile zero behind it, so that
    // after the next barrier the decode starts at once.  Items come from the
    // launch's ticket counter, so that workgroups that run faster take more
    // of them.
    u32x4 cw[kCodeLoads];
    u32x2 rw[kBlocks];
    u32x4 lr[kLutLoads];
    // The current item (the first is the workgroup's number).  Every wave
    // reads an item's record itself, with one scalar load, so records need
    // no LDS slot and no barrier of their own.
    uint32_t cur = blockIdx.x;
    WinScan sc;
    {
        const Item it = item_at(a, min(cur, n - 1));
        const uint32_t win = load_windows(it, tid);
        load_codes(it, tid, cw);
        load_lut(a, it.lut, tid, lr);
        // At the start every workgroup requests its first chunk at once: the
        // raw bytes are requested only once the code bytes are in, so that
        // the code bytes come first and the raw bytes load during the first
        // decode (0.8% faster overall).
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) rw[b] = load_raw(it, tid, b);
        // the tile starts zero; from then on each assembly clears what it read
#pragma unroll
        for (uint32_t i = 0; i < sizeof(L.tile) / 16; i += kThreads)
            if (i + tid < sizeof(L.tile) / 16) reinterpret_cast<u32x4 *>(L.tile)[i + tid] = u32x4{0u, 0u, 0u, 0u};
        if (it.staged) stage_codes(L, tid, cw);
        put_lut(L, tid, lr);
        sc = scan_windows(L, it, win, tid, lane, wave, 0);
    }

    for (uint32_t k = 0;; ++k) {
        // ---- the previous item's tile is read and cleared; this item's
        //      code bytes, tables and wave totals are in LDS
        __syncthreads();
        const uint32_t sl = k & 1u;
        if (cur >= n) break;
        // The next chunk's ticket is taken once this chunk is decoded, so
        // that at the end of the launch no workgroup holds a chunk in reserve
        // while others have run out (about 3% faster than taking it one chunk
        // ahead); only a workgroup's first chunk takes it before decoding,
        // when every workgroup would otherwise wait for it at once.  Wave 0
        // takes it and leaves it in LDS for the barrier that ends the decode.
        // (A ticket of n or above: no item; the next item's loads then read
        // item n-1's bytes, so that they stay unconditional and the compiler
        // can count them and wait for the oldest ones only.)
        const bool late = k != 0;
        const Item it = item_at(a, cur);
        if (wave == 0 && !late) {
            const uint32_t t1 = take_ticket(a, lane);
            if (lane == 0) L.rec_id[sl ^ 1u] = t1;
        }

        // ---- windows 2*tid (a) and 2*tid+1 (b): output positions
        const uint32_t b1 = it.rel0 + it.nbits;
        const uint32_t nc = it.nc;
        uint32_t na = sc.na, nb = sc.nb;
        const uint32_t sa = sc.sa, sb = sc.sb;
        uint32_t base = 0;
        for (uint32_t w = 0; w < wave; ++w) base += L.wave_total[sl][w];
        const uint32_t qa = base + sc.incl - na - nb;
        const uint32_t qb = qa + na;
        // never write past the chunk, whatever the device bytes say
        uint32_t bad = 0;
        {
            const uint32_t ca = qa < nc ? min(na, nc - qa) : 0u;
            const uint32_t cb = qb < nc ? min(nb, nc - qb) : 0u;
            bad |= (ca != na) | (cb != nb);
            na = ca;
            nb = cb;
        }
        // Peeks at p <= pmax stay inside the source.  A start past pmax:
        // only a container that disagrees with its index (valid starts lie
        // before the chunk's last bit, and the stream's 16 bytes of padding
        // and the staging area keep that below pmax).
        const uint32_t pmax = it.staged ? 32u * (kCodeWords - 1) : 32u * (it.n_words - 1);
        bad |= (sa > pmax) | (sb > pmax);
        const uint32_t pa = min(sa, pmax), pb = min(sb, pmax);
        // T counted look-ups: while no window of the wave can run out of
        // codes before its last counted look-up (a look-up takes at most
        // three) and no peek can pass pmax (a look-up moves a window at most
        // 24 bits; a bound on T alone, 24 T below pmax for every start, would
        // move the valid starts of chunks that end near pmax)
        const uint32_t room = (pmax - max(pa, pb)) / 24u;
        const uint32_t m = min(na, nb);
        // (staged codes: the last counted look-up may take a window's last
        // codes, since its entry is kept; codes in global memory: it may not)
        const uint32_t Tm = m == 0 ? 0u : it.staged ? (m - 1) / kMaxPerLookup + 1 : (m - 1) / kMaxPerLookup;
        const uint32_t T = __builtin_amdgcn_readfirstlane(wave_min(min(Tm, room)));
        Chain A{pa + kPosBias, qa << 3, qa + na, 0u};
        Chain B{pb + kPosBias, qb << 3, qb + nb, 0u};
        if (it.staged) {
            // code-word reads: codes[k .. k+2] with k = P / 32 <= kCodeWords - 1
            const LdsCodes src{L.codes, pmax + kPosBias};
            decode_pair(L, src, A, B, T, bad);
        } else {
            // peeks read words k-1 and k of the stream from s0, k < n_words
            const GlobalCodes src{reinterpret_cast<const GLOBAL uint32_t *>(it.stream) - 1, pmax + kPosBias};
            decode_pair(L, src, A, B, T, bad);
        }
        const uint32_t ea = A.P - kPosBias;
        const uint32_t eb = B.P - kPosBias;
        // (the ticket's round trip overlaps the wait for the other waves)
        if (wave == 0 && late) {
            const uint32_t t1 = take_ticket(a, lane);
            if (lane == 0) L.rec_id[sl ^ 1u] = t1;
        }
        __syncthreads();
        const uint32_t nid = __builtin_amdgcn_readfirstlane(L.rec_id[sl ^ 1u]);

        // ---- every non-empty window ends where the next non-empty window's
        //      first code starts; the last one at the chunk end
        {
            const uint64_t above = lane == 63 ? 0 : (sc.mask >> (lane + 1));
            const uint32_t nxt_lane = above ? lane + 1 + (uint32_t)__builtin_ctzll(above) : lane;
            const uint32_t nxt_first = __shfl(sc.first, (int)nxt_lane);
            uint32_t after_b = b1;
            if (above) {
                after_b = nxt_first;
            } else {
                for (uint32_t w = wave + 1; w < (uint32_t)kWaves; ++w) {
                    const uint32_t f = L.wave_first[sl][w];
                    if (f != 0xFFFFFFFFu) {
                        after_b = f;
                        break;
                    }
                }
            }
            if (nb) bad |= eb != after_b;
            if (na) bad |= ea != (nb ? sb : after_b);
            bad_any |= bad;
        }

        // ---- assemble and store the whole 2048-element blocks, clearing
        //      the tile dwords read; each block's raw registers take the next
        //      item's bytes right after use.  The next item's window entries,
        //      code bytes and tables are requested first: they are needed
        //      first.
        // (the assembly issues all of the kernel's memory traffic, the
        // decode only VALU and LDS work: a wave assembling goes first, so
        // that the compute unit's other waves' decodes do not hold back its
        // loads and stores; about 1% faster)
        __builtin_amdgcn_s_setprio(3);
        const Item nx = item_at(a, min(nid, n - 1));
        const uint32_t win_nx = load_windows(nx, tid);
        load_codes(nx, tid, cw);
        load_lut(a, nx.lut, tid, lr);
        GLOBAL uint16_t *o = it.out;
        const uint32_t full = nc / kBlockElems;
        // the tile offset of this lane's two dwords in block 0; block b's are
        // tile_off(512 b + 2 tid) = 2112 b + that
        const uint32_t tb0 = tile_off(2u * tid);
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
            if ((uint32_t)b < full) {
                uint32_t *tp = reinterpret_cast<uint32_t *>(L.tile + tb0 + 2112u * b);
                const u32x2 t8{tp[0], tp[1]};
                tp[0] = 0u;
                tp[1] = 0u;
                GLOBAL u32x4 *ob = uniform(reinterpret_cast<GLOBAL u32x4 *>(o + kBlockElems * b));
                __builtin_nontemporal_store(join8(t8, rw[b]), ob + tid);
            }
            rw[b] = load_raw(nx, tid, b);
        }
        if (nc < (uint32_t)kChunk) {
            // ---- the ragged last block of a tensor (raw bytes fetched again)
            const uint32_t j = full * kBlockElems + 8 * tid;
            if (j < nc) {
                const u32x2 r8 = *reinterpret_cast<const GLOBAL u32x2 *>(it.raw + j);   // j + 8 <= raw bytes
                uint32_t *tp = reinterpret_cast<uint32_t *>(L.tile + tile_off(j >> 2));   // j/4 even: +4 is dword j/4 + 1
                const u32x2 t8{tp[0], tp[1]};
                tp[0] = 0u;
                tp[1] = 0u;
                const u32x4 v = join8(t8, r8);
                if (j + 8 <= nc) {
                    *reinterpret_cast<GLOBAL u32x4 *>(o + j) = v;
                } else {
                    for (uint32_t k = 0; j + k < nc; ++k) {
                        const uint32_t wd = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
                        o[j + k] = (uint16_t)(wd >> (16 * (k & 1)));
                    }
                }
            }
            // a window's last look-up and spill reach at most 6 elements past
            // the chunk's end: clear the dwords the ragged block did not
            if (tid < 3u) {
                const uint32_t d = ((nc + 7u) >> 3) * 2u + tid;
                *reinterpret_cast<uint32_t *>(L.tile + tile_off(d)) = 0u;
            }
        }
        // the next item: its tables and staged code bytes (nothing reads
        // them after the decode) and its window scan
        put_lut(L, tid, lr);
        if (nx.staged) stage_codes(L, tid, cw);
        sc = scan_windows(L, nx, win_nx, tid, lane, wave, sl ^ 1u);
        cur = nid;
        __builtin_amdgcn_s_setprio(0);
    }
    if (__ballot(bad_any) && lane == 0) atomicOr(a.status, 1u);
    // The last workgroup to finish (every ticket of the launch has been
    // taken by then) clears the counter for the slot's next launch, then
    // tells the host the slot is free.
    if (tid == 0 && atomicAdd(a.work + 1, 1u) == gridDim.x - 1) {
        atomicExch(a.work, 0u);
        atomicExch(a.work + 1, 0u);
        // The host may give the slot to a new launch once it reads the id,
        // so the two resets must be done first: wait for them (vmcnt counts
        // them until they are performed), then store the id.  A release at
        // system scope would order them too, but it writes back the whole
        // L2 first, at the end of every launch.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __hip_atomic_store(a.fin, a.launch_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

hipError_t launch_decode(const DecodeArgs &args, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(kThreads), 0, stream, args);
    return hipGetLastError();
}

int decode_wgs_per_cu() {
    static int cached = 0;
    if (!cached) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel, kThreads, 0) != hipSuccess || n <= 0) n = 1;
        cached = n;
    }
    return cached;
}

}  // namespace df11
