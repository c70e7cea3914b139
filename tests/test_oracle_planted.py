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
    ("window gap off by one",
     "gap[win] = (unsigned)(p - (b0 + window_edge(b1 - b0, win)));",
     "gap[win] = (unsigned)(p - (b0 + window_edge(b1 - b0, win)) + 1);", 0),
    ("window entry packs the gap one bit low",
     "(uint16_t)(cnt[i] | (gap[i] << 11))", "(uint16_t)(cnt[i] | (gap[i] << 10))", 0),
    ("window count misses a code that starts on the window's first bit",
     "            cnt[win]++;",
     "            cnt[win] += (p != b0 + window_edge(b1 - b0, win));", 0),
    ("window edges round up",
     "return i * N / WINDOWS;", "return (i * N + WINDOWS - 1) / WINDOWS;", 0),
    ("window search stops one window early",
     "while (win + 1 < WINDOWS && b0 + window_edge(b1 - b0, win + 1) <= p) win++;",
     "while (win + 1 < WINDOWS && b0 + window_edge(b1 - b0, win + 1) < p) win++;", 0),
    ("chunk start bit recorded after the first code",
     "put_u64(out + L.off_ci + (j / CHUNK) * 16, pos);",
     "put_u64(out + L.off_ci + (j / CHUNK) * 16, pos + 1);", 0),
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
            # the index from first principles: code starts from the source
            # and the header's code lengths, windows at floor(i * N / 512)
            h = oracle.header(c)
            ci = c[h["off_chunk_index"]:h["off_chunk_index"] + 16 * (h["n_chunks"] + 1)].view(np.uint64)
            b0, b1 = int(ci[2 * ch]), int(ci[2 * ch + 2])
            ln = h["code_len"].astype(np.int64)[(w[lo:hi] >> 7) & 0xFF]
            starts = b0 + np.concatenate([[0], np.cumsum(ln)[:-1]])
            NW = oracle.WINDOWS
            edges = b0 + (np.arange(NW) * (b1 - b0)) // NW
            before = np.searchsorted(starts, edges, side="left")
            want_cnt = np.diff(np.append(before, hi - lo))
            ent = c[h["off_windows"] + 2 * NW * ch:h["off_windows"] + 2 * NW * (ch + 1)].view(np.uint16)
            cnt, gap = ent & 0x7FF, ent >> 11
            want_gap = np.where(want_cnt > 0, starts[np.minimum(before, hi - lo - 1)] - edges, 0)
            if not ((cnt == want_cnt).all() and (gap == want_gap).all()):
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
