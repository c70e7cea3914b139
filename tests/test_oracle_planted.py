"""The oracle's pins have teeth: a plausible mistake planted in a copy of the
oracle's C source (a dropped term, a wrong shift, an off-by-one index, a
flipped bit order, a wrong comparison) makes at least one pin fail.

Mistakes are planted on the CPU only, in a temporary copy; the oracle under
`oracle/` is never modified."""
import hashlib
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import tiny
from lossless_bf16_weight_amd import workloads as W

SRC = os.path.join(os.path.dirname(oracle.__file__), "df11_oracle.c")
HDR = os.path.join(os.path.dirname(oracle.__file__), "df11_oracle.h")

# (name, text in df11_oracle.c, replacement, which occurrence (0 = first))
MUTATIONS = [
    ("raw byte takes the wrong sign bit",
     "return ((w >> 8) & 0x80u) | (w & 0x7Fu);", "return ((w >> 9) & 0x80u) | (w & 0x7Fu);", 0),
    ("exponent field shifted by one",
     "return (w >> 7) & 0xFFu;", "return (w >> 8) & 0xFFu;", 0),
    ("package-merge keeps one item too few",
     "for (int i = 0; i < 2 * n - 2; i++)", "for (int i = 0; i < 2 * n - 3; i++)", 0),
    ("package weight drops a term",
     "pk.weight = a->weight + b->weight;", "pk.weight = a->weight;", 0),
    ("canonical code forgets the increment",
     "c = (c + 1) << (len[order[i]] - len[order[i - 1]]);",
     "c = c << (len[order[i]] - len[order[i - 1]]);", 0),
    ("stream written least significant bit first",
     "stream[pos / 8] |= (uint8_t)(0x80u >> (pos % 8));",
     "stream[pos / 8] |= (uint8_t)(0x01u << (pos % 8));", 0),
    ("both bit writer and reader least significant bit first",
     None, None, 0),
    ("window length misses its last code",
     "for (uint64_t i = 0; i < WCODES; i++) bits += len[exponent_of(words[c * CHUNK + k * WCODES + i])];",
     "for (uint64_t i = 0; i + 1 < WCODES; i++) bits += len[exponent_of(words[c * CHUNK + k * WCODES + i])];", 0),
    ("window base is the first window's length, not the smallest",
     "if (!any || bits < lo) lo = bits;", "if (!any) lo = bits;", 0),
    ("the chunk's last window gets an entry",
     "        for (uint64_t k = 0; k + 1 < nw; k++) {\n            uint64_t e = wbits[c * WINDOWS + k] - lo;",
     "        for (uint64_t k = 0; k < nw && k < WINDOWS - 1; k++) {\n            uint64_t e = wbits[c * WINDOWS + k] - lo;", 0),
    ("window decoder starts one window late",
     "for (int k = 0; k < win && (uint64_t)k + 1 < nw; k++)",
     "for (int k = 0; k <= win && (uint64_t)k + 1 < nw; k++)", 0),
    ("window decoder leaves out the base",
     "pos += P.base + get_entry(c, &P.L, chunk, (uint64_t)k);",
     "pos += get_entry(c, &P.L, chunk, (uint64_t)k);", 0),
    ("windows of 63 codes in the decoder",
     "uint64_t j0 = chunk * CHUNK + (uint64_t)win * WCODES;",
     "uint64_t j0 = chunk * CHUNK + (uint64_t)win * (WCODES - 1);", 0),
    ("chunk start bit recorded after the first code",
     "if (j % CHUNK == 0) put_u64(out + L.off_ci + (j / CHUNK) * 8, pos);",
     "if (j % CHUNK == 0) put_u64(out + L.off_ci + (j / CHUNK) * 8, pos + 1);", 0),
    ("decoder accepts one code too many per length",
     "v - P->first[k] < P->count[k]", "v - P->first[k] <= P->count[k]", 0),
    ("decoder joins the exponent one bit too high",
     "((e & 0xFFu) << 7)", "((e & 0xFFu) << 8)", 0),
    ("leaves sorted by symbol only",
     "(freq[sym[j]] > freq[s] || (freq[sym[j]] == freq[s] && sym[j] > s))",
     "(sym[j] > s)", 0),
    ("SHA-256 schedule rotates by 8 instead of 7",
     "rotr(w[t - 15], 7)", "rotr(w[t - 15], 8)", 0),
    ("SHA-256 round constants from square roots",
     "S->k[i] = (uint32_t)iroot((unsigned __int128)p[i] << 96, 3);",
     "S->k[i] = (uint32_t)iroot((unsigned __int128)p[i] << 64, 2);", 0),
    ("SHA-256 length field in bytes",
     "uint64_t bits = S->length * 8;", "uint64_t bits = S->length;", 0),
    ("SHA-256 majority replaced by choice",
     "uint32_t maj = (a & b) ^ (a & c) ^ (b & c);", "uint32_t maj = (a & b) ^ (~a & c);", 0),
    ("source words hashed high byte first",
     "sha256_byte(&S, (uint8_t)(w[j] & 0xFFu));\n        sha256_byte(&S, (uint8_t)(w[j] >> 8));",
     "sha256_byte(&S, (uint8_t)(w[j] >> 8));\n        sha256_byte(&S, (uint8_t)(w[j] & 0xFFu));", 0),
]


def _pins_pass() -> bool:
    """A compact battery of the pins; False as soon as one fails."""
    try:
        # SHA-256 against hashlib around the padding boundaries, and the
        # source hash of a container against hashlib of the words' bytes
        for n in (0, 3, 55, 56, 64, 119, 1000):
            b = bytes(range(256)) * 4
            if oracle.sha256(b[:n]) != hashlib.sha256(b[:n]).digest():
                return False
        w = W.normal_bf16((5000,), seed=2)
        c = oracle.encode(w, sha256=True)
        if oracle.header(c)["sha256"] != hashlib.sha256(w.astype("<u2").tobytes()).digest():
            return False
        if oracle.check(c) != 0:
            return False
        # golden BF16 fields and the exhaustive tensor
        w = W.exhaustive_words()
        c = oracle.encode(w)
        if oracle.check(c) != 0 or not (oracle.decode(c, w.size) == w).all():
            return False
        h = oracle.header(c)
        raw = c[h["off_raw"]:h["off_raw"] + w.size]
        if not (raw == (((w >> 15).astype(np.uint8) << 7) | (w & 0x7F).astype(np.uint8))).all():
            return False
        if tiny.decode_with_strings(c.tobytes()) != w.tolist():
            return False
        # textbook example and brute-force optimality
        f = np.zeros(256, np.uint64)
        f[:6] = [45, 13, 12, 16, 9, 5]
        if int((f * oracle.code_lengths(f)).sum()) != 224:
            return False
        for seed in range(8):
            rng = np.random.default_rng(seed)
            k = int(rng.integers(2, 8))
            f = np.zeros(256, np.uint64)
            f[rng.choice(256, k, replace=False)] = (rng.pareto(1.0, k) * 50 + 1).astype(np.uint64)
            ln = oracle.code_lengths(f, 5)
            if sum(1 << (24 - int(l)) for l in ln if l) != 1 << 24:
                return False
            if int((f * ln).sum()) != tiny.brute_force_min_cost(f.tolist(), 5):
                return False
            code = oracle.canonical_codes(ln)
            strings = {s: format(int(code[s]), "0%db" % int(ln[s])) for s in range(256) if ln[s]}
            if tiny.canonical_code_strings([int(x) for x in ln]) != strings:
                return False
        # Gaussian tensor with a ragged tail: index, windows, sampled chunks
        w = W.normal_bf16((2 * 32768 + 777,), seed=4)
        c = oracle.encode(w)
        if oracle.check(c) != 0 or not (oracle.decode(c, w.size) == w).all():
            return False
        if tiny.decode_with_strings(c.tobytes()) != w.tolist():
            return False
        for ch in range(3):
            lo, hi = ch * 32768, min(w.size, (ch + 1) * 32768)
            if not (oracle.decode_chunk(c, ch, hi - lo) == w[lo:hi]).all():
                return False
            parts = [oracle.decode_window(c, ch, win)[0] for win in range(oracle.WINDOWS)]
            if not (np.concatenate(parts) == w[lo:hi]).all():
                return False
            # the index from first principles: chunk start bits are the
            # cumulative code lengths; window entries the lengths of
            # 64-code groups (all but the chunk's last) minus the smallest
            h = oracle.header(c)
            ln = h["code_len"].astype(np.int64)[(w >> 7) & 0xFF]
            cum = np.concatenate([[0], np.cumsum(ln)])
            ci = c[h["off_chunk_index"]:h["off_chunk_index"] + 8 * (h["n_chunks"] + 1)].view(np.uint64)
            if not (ci == cum[np.minimum(np.arange(h["n_chunks"] + 1) * 32768, w.size)]).all():
                return False
            groups = []
            for c0 in range(0, w.size, 32768):
                seg = ln[c0:c0 + 32768]
                nw = (seg.size + 63) // 64
                groups.append(seg[:64 * (nw - 1)].reshape(-1, 64).sum(axis=1))
            base = int(np.concatenate(groups).min())
            if h["window_base"] != base or h["entry_bytes"] != 1:
                return False
            NW = oracle.WINDOWS
            ent = c[h["off_windows"] + NW * ch:h["off_windows"] + NW * (ch + 1)].astype(np.int64)
            g = groups[ch]
            if not ((ent[:g.size] == g - base).all() and (ent[g.size:] == 0).all()):
                return False
        return True
    except Exception:
        return False


def _build_mutant(tmp, name, old, new, which):
    src = open(SRC).read()
    if old is None:  # consistent LSB-first writer and reader
        pairs = [("stream[pos / 8] |= (uint8_t)(0x80u >> (pos % 8));",
                  "stream[pos / 8] |= (uint8_t)(0x01u << (pos % 8));"),
                 ("return (stream[pos / 8] >> (7 - pos % 8)) & 1u;",
                  "return (stream[pos / 8] >> (pos % 8)) & 1u;")]
    else:
        pairs = [(old, new)]
    for o, n in pairs:
        assert src.count(o) > which, f"mutation site not found: {o}"
        idx = -1
        for _ in range(which + 1):
            idx = src.index(o, idx + 1)
        src = src[:idx] + n + src[idx + len(o):]
    d = os.path.join(tmp, str(abs(hash(name))))
    os.makedirs(d)
    shutil.copy(HDR, d)
    with open(os.path.join(d, "df11_oracle.c"), "w") as f:
        f.write(src)
    so = os.path.join(d, "libmutant.so")
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", "-o", so,
                           os.path.join(d, "df11_oracle.c")])
    return so


def test_unmutated_oracle_passes_the_battery():
    assert _pins_pass()


@pytest.mark.parametrize("name,old,new,which", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, which):
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(tmp, name, old, new, which)
        with oracle.use_library(so):
            assert not _pins_pass(), f"planted mistake not caught: {name}"
