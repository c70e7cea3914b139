// Sanitizer driver for the host code of libdf11 (validation, encoders, SHA-256,
// NF12 host code), built with clang++ -fsanitize=address,undefined on the CPU.
//
// Reads a manifest of "<kind> <path>" lines:
//   slots -                 the decode's ticket-counter slots (SlotTable)
//   luts  -                 the decode tables against the kernel's look-up arithmetic
//   df11  <container file>  df11_validate on the whole file and on prefixes
//   nf12  <container file>  df11_nf12_validate on the whole file and on prefixes
//   words <16-bit words>    df11_encode (1 and 4 threads), df11_encode_ex with the
//                           source hash, df11_validate and df11_verify_words on
//                           the result, df11_nf12_encode + validate; the DF11
//                           container is written to <path>.asan.df11
// Any memory error or undefined behaviour aborts with the sanitizer's report;
// a status that contradicts the input's kind exits 3.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "df11.h"
#include "df11_internal.hpp"
#include "nf12_internal.hpp"

// The kernels are not part of this build: the driver never plans or decodes.
namespace df11 {
hipError_t launch_decode(const DecodeArgs &, int, hipStream_t) { abort(); }
int decode_wgs_per_cu() { abort(); }
hipError_t launch_bw_control(const void *, uint64_t, void *, uint64_t, int, hipStream_t) { abort(); }
hipError_t launch_nf12_decode(const Nf12Args &, int, hipStream_t) { abort(); }
}  // namespace df11

static std::vector<uint8_t> read_file(const char *path) {
    std::vector<uint8_t> b;
    FILE *f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(2);
    }
    uint8_t buf[1 << 16];
    size_t k;
    while ((k = fread(buf, 1, sizeof buf, f)) > 0) b.insert(b.end(), buf, buf + k);
    fclose(f);
    return b;
}

// Validates prefixes of a container; each copy is exactly as long as the
// prefix, so a read past it is a heap overflow the sanitizer reports.
template <class F>
static void prefixes(const std::vector<uint8_t> &c, F validate) {
    const size_t cuts[] = {0, 1, 8, 16, 100, 255, 256, 511, 512, 513, 1024, 4096, c.size() / 3, c.size() / 2,
                           c.size() > 0 ? c.size() - 1 : 0, c.size()};
    for (size_t n : cuts) {
        if (n > c.size()) continue;
        std::vector<uint8_t> p(c.begin(), c.begin() + n);
        validate(p.empty() ? nullptr : p.data(), n);
    }
}

static int check_words(const char *path) {
    std::vector<uint8_t> raw = read_file(path);
    const uint64_t n = raw.size() / 2;
    std::vector<uint16_t> w(n);
    if (n) memcpy(w.data(), raw.data(), 2 * n);
    const uint64_t dims[1] = {n};
    const uint64_t cap = df11_container_bound(n);
    std::vector<uint8_t> a(cap), b(cap), h(cap);
    uint64_t na = 0, nb = 0, nh = 0;
    if (df11_encode(w.data(), n, 1, dims, a.data(), cap, &na, 1) != DF11_OK) return 3;
    if (df11_encode(w.data(), n, 1, dims, b.data(), cap, &nb, 4) != DF11_OK) return 3;
    if (na != nb || memcmp(a.data(), b.data(), na) != 0) return 3;
    if (df11_encode_ex(w.data(), n, 1, dims, DF11_FLAG_SHA256, h.data(), cap, &nh, 3) != DF11_OK) return 3;
    if (nh != na) return 3;
    df11_tensor_info info;
    if (df11_validate(a.data(), na, &info) != DF11_OK || info.n_elems != n) return 3;
    if (df11_validate(h.data(), nh, &info) != DF11_OK) return 3;
    if (df11_verify_words(h.data(), nh, w.data(), n) != DF11_OK) return 3;
    if (df11_verify_words(a.data(), na, w.data(), n) != DF11_E_UNSUPPORTED) return 3;
    // a container smaller than the bound: the encoder must refuse, not overrun
    if (na > 1 && df11_encode(w.data(), n, 1, dims, b.data(), na - 1, &nb, 2) == DF11_OK) return 3;
    const uint64_t ncap = df11_nf12_bound(n);
    std::vector<uint8_t> f(ncap ? ncap : 1);
    uint64_t nf = 0;
    if (df11_nf12_encode(w.data(), n, f.data(), ncap, &nf, 2) != DF11_OK) return 3;
    uint64_t ne = 0;
    if (df11_nf12_validate(f.data(), nf, &ne) != DF11_OK || ne != n) return 3;
    std::string out = std::string(path) + ".asan.df11";
    FILE *o = fopen(out.c_str(), "wb");
    if (!o || fwrite(a.data(), 1, na, o) != na) return 2;
    fclose(o);
    return 0;
}

// The host side of the decode's ticket-counter slots (SlotTable): no slot is
// given out while the device has not reported its previous launch finished,
// captured launches keep theirs, a failed launch gives its slot back.
static int check_slots() {
    using df11::kWorkSlots;
    df11::SlotTable T;
    uint32_t fin[kWorkSlots] = {};
    uint32_t id = 0, ids[kWorkSlots];
    bool seen[kWorkSlots] = {};
    for (uint32_t i = 0; i < kWorkSlots; ++i) {
        const int s = T.acquire(fin, false, &id);
        if (s < 0 || seen[s] || id == 0) return 10;
        seen[s] = true;
        ids[s] = id;
    }
    if (T.acquire(fin, false, &id) >= 0) return 11;          // all held
    fin[7] = ids[7];                                          // slot 7's launch finished
    if (T.acquire(fin, false, &id) != 7 || id == ids[7]) return 12;
    ids[7] = id;
    if (T.acquire(fin, false, &id) >= 0) return 13;
    fin[9] = ids[9] - 1;                                      // an older id: still running
    if (T.acquire(fin, false, &id) >= 0) return 14;
    fin[9] = ids[9];
    if (T.acquire(fin, true, &id) != 9) return 15;           // captured: kept for good
    fin[9] = id;
    if (T.acquire(fin, false, &id) >= 0) return 16;
    // once every launch has finished, every slot but the captured one comes
    // back, each once before any comes back twice
    for (uint32_t s = 0; s < kWorkSlots; ++s) fin[s] = T.issued[s];
    bool back[kWorkSlots] = {};
    for (uint32_t i = 0; i + 1 < kWorkSlots; ++i) {
        const int s = T.acquire(fin, false, &id);
        if (s < 0 || s == 9 || back[s]) return 18;
        back[s] = true;
    }
    if (T.acquire(fin, false, &id) >= 0) return 17;          // all held again
    // a launch call that failed gives its slot back at once
    for (uint32_t s = 0; s < kWorkSlots; ++s) fin[s] = 0;
    df11::SlotTable U;
    const int a = U.acquire(fin, false, &id);
    U.release(a);
    if (U.acquire(fin, false, &id) < 0) return 19;
    // captured launches: at most half of the slots
    df11::SlotTable V;
    int n_cap = 0;
    while (V.acquire(fin, true, &id) >= 0) ++n_cap;
    if (n_cap != (int)df11::kGraphSlotsMax || V.acquire(fin, false, &id) < 0) return 20;
    return 0;
}

// The decode tables (build_lut) against the kernel's look-up arithmetic, on
// random streams for many codes: a first-level entry by the next 10 bits,
// a subtable entry at l2 - 2 + F + bfe(peek, 11, k + 1) for a prefix whose
// first code is longer, the canonical limits for codes longer than 16 bits.
// Every look-up must give the next codes' exponents and bits as the
// canonical code (from the encoder's own construction) has them.
static uint64_t lcg(uint64_t &x) {
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    return x >> 33;
}

static int check_luts() {
    using namespace df11;
    uint64_t rng = 12345;
    for (int trial = 0; trial < 400; ++trial) {
        uint64_t freq[256] = {};
        const int kind = trial % 5;
        const int nsym = kind == 3 ? 1 + trial % 3 : 1 + (int)(lcg(rng) % 256);
        for (int i = 0; i < nsym; ++i) {
            const int sym = (int)(lcg(rng) % 256);
            uint64_t f = 1;
            if (kind == 0) f = 1 + (uint64_t)(1e9 / (1.0 + (double)i * i));     // peaked
            if (kind == 1) f = (uint64_t)1 << (i % 40);                         // up to the 24-bit cap
            if (kind == 2) f = 1 + lcg(rng) % 1000;                             // flat
            if (kind == 4) f = i < 6 ? 1000000000ull : 1 + lcg(rng) % 3;        // heavy tail
            freq[sym] += f;
        }
        uint8_t len[256];
        uint32_t code[256];
        build_code(freq, len, code);
        LutRecord R;
        build_lut(len, R);
        int syms[256], n = 0;
        for (int e = 0; e < 256; ++e)
            if (len[e]) syms[n++] = e;
        // a stream of 3000 codes, symbols drawn uniformly (long codes often)
        std::vector<uint8_t> bits = {0, 0};   // two bits before the stream
        std::vector<int> seq;
        for (int i = 0; i < 3000; ++i) {
            const int e = syms[lcg(rng) % (uint64_t)n];
            seq.push_back(e);
            for (int b = len[e] - 1; b >= 0; --b) bits.push_back((uint8_t)((code[e] >> b) & 1));
        }
        for (int i = 0; i < 64; ++i) bits.push_back((uint8_t)(lcg(rng) & 1));
        size_t p = 2, i = 0;
        while (i < seq.size()) {
            uint32_t ta = 0;
            for (int b = 0; b < 32; ++b) ta |= (uint32_t)bits[p - 2 + b] << b;
            uint32_t ent = R.l1[(ta >> 2) & (kL1Size - 1)];
            if ((ent >> kEntCountShift) == 0) {
                const uint32_t w = ent & 31u;
                const uint32_t ia = (ent >> 16) + ((ta >> 11) & ((1u << w) - 1u));
                if (ia < 2 || (ia & 1u) || (ia - 2) / 2 >= (uint32_t)kL2Max) return 30;
                const uint32_t ra = R.l2[(ia - 2) / 2];
                if (ra) {
                    ent = (ra & 0xFFu) | ((ra >> 8) << 24);
                } else {
                    const uint32_t v = __builtin_bitreverse32(ta >> 2) >> (32 - kMaxLen);
                    uint32_t l = kL1Bits + 1;
                    while (l <= (uint32_t)kMaxLen && v >= R.lim[l]) ++l;
                    if (l > (uint32_t)kMaxLen) return 31;
                    ent = R.sorted[(int)(v >> (kMaxLen - l)) + R.base[l]] | (l << kEntLenShift) | (1u << kEntCountShift);
                }
            }
            const uint32_t cnt = ent >> kEntCountShift, nb = (ent >> kEntLenShift) & 31u;
            if (cnt == 0 || cnt > (uint32_t)kMaxPerLookup) return 32;
            uint32_t used = 0;
            for (uint32_t j = 0; j < cnt && i < seq.size(); ++j, ++i) {
                if (((ent >> (8 * j)) & 0xFFu) != rot_exp((unsigned)seq[i])) return 33;
                used += len[seq[i]];
            }
            if (i < seq.size() && used != nb) return 34;
            p += nb;
        }
    }
    return 0;
}

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s MANIFEST\n", argv[0]);
        return 2;
    }
    FILE *m = fopen(argv[1], "r");
    if (!m) return 2;
    char kind[16], path[4096];
    long n_df11 = 0, n_nf12 = 0, n_words = 0;
    while (fscanf(m, "%15s %4095s", kind, path) == 2) {
        if (!strcmp(kind, "df11")) {
            const std::vector<uint8_t> c = read_file(path);
            prefixes(c, [](const uint8_t *p, size_t n) {
                df11_tensor_info info;
                (void)df11_validate(p, n, &info);
                (void)df11_validate(p, n, nullptr);
            });
            ++n_df11;
        } else if (!strcmp(kind, "nf12")) {
            const std::vector<uint8_t> c = read_file(path);
            prefixes(c, [](const uint8_t *p, size_t n) {
                uint64_t ne;
                (void)df11_nf12_validate(p, n, &ne);
            });
            ++n_nf12;
        } else if (!strcmp(kind, "slots")) {
            const int r = check_slots();
            if (r) {
                fprintf(stderr, "slot table check %d failed\n", r);
                return 3;
            }
        } else if (!strcmp(kind, "luts")) {
            const int r = check_luts();
            if (r) {
                fprintf(stderr, "decode table check %d failed\n", r);
                return 3;
            }
        } else if (!strcmp(kind, "words")) {
            const int r = check_words(path);
            if (r) {
                fprintf(stderr, "words %s: status %d\n", path, r);
                return r;
            }
            ++n_words;
        } else {
            return 2;
        }
    }
    fclose(m);
    printf("ok: %ld df11, %ld nf12, %ld word files\n", n_df11, n_nf12, n_words);
    return 0;
}
