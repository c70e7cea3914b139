"""Pins of the NF12 oracle (oracle/nf12_oracle.c) to what the page and the
BF16 format fix, not to itself.

Source: the nf12 news page ("Developer open-sources nf12: lossless 12-bit
compression for BF16 models"), "How it works" (the top four exponent bits
0111 are dropped and restored) and "Implementation details" (groups of 8, 16
bytes packed into 12, outlier groups flagged and kept whole in an escape
buffer, 28 bytes per escaped group)."""
import math
import os

import numpy as np
import pytest

from oracle import nf12, tiny
from lossless_bf16_weight_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split("#")[0].strip() for ln in f if ln.split("#")[0].strip()]


def test_golden_fields():
    rows = _rows("nf12_fields.txt")
    assert len(rows) == 14
    for r in rows:
        word, fits, code = r.split()[:3]
        w = int(word, 16)
        assert nf12.fits(w) == (fits == "1"), word
        if fits == "1":
            assert nf12.code(w) == int(code, 16), word
            assert nf12.word(int(code, 16)) == w, word


def test_golden_group_slots():
    for r in _rows("nf12_groups.txt"):
        left, right = r.split("|")
        words = np.array([int(x, 16) for x in left.split()], np.uint16)
        want = bytes(int(x, 16) for x in right.split())
        c = nf12.encode(words)
        h = nf12.header(c)
        assert h["n_groups"] == 1 and h["n_escaped"] == 0
        assert c[h["off_slots"]:h["off_slots"] + 12].tobytes() == want
        assert (nf12.decode(c, 8) == words).all()


def test_fits_is_the_top_four_exponent_bits():
    """Every one of the 65,536 words: it fits exactly when bits 14..11 are
    0111, and its code decodes back to it."""
    w = np.arange(65536, dtype=np.uint32)
    top4 = (w >> 11) & 0xF
    for x in range(65536):
        assert nf12.fits(x) == (top4[x] == 7)
        if top4[x] == 7:
            c = nf12.code(x)
            assert c < 4096 and nf12.word(c) == x
    # 4096 codes, one word each (both signs x 16 exponents x 128 fractions)
    assert int((top4 == 7).sum()) == 4096


def test_exhaustive_words_round_trip():
    w = W.exhaustive_words()
    c = nf12.encode(w)
    assert nf12.check(c) == 0
    assert (nf12.decode(c, w.size) == w).all()
    h = nf12.header(c)
    # in counting order, a group of 8 fits only inside the two runs of 2048
    # words whose top exponent bits are 0111 (0x3800-0x3fff, 0xb800-0xbfff)
    assert h["n_groups"] == 8192 and h["n_escaped"] == 8192 - 2 * 2048 // 8


@pytest.mark.parametrize("n", [0, 1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 511, 512, 513, 4095, 4097])
def test_sizes_round_trip_and_match_the_second_implementation(n):
    rng = np.random.default_rng(n)
    w = rng.integers(0x3700, 0x4080, n).astype(np.uint16)     # mostly fitting, some not
    c = nf12.encode(w)
    assert nf12.check(c) == 0
    assert (nf12.decode(c, n) == w).all()
    if n <= 1024:
        assert c.tobytes() == tiny.nf12_encode_tiny([int(x) for x in w])


def test_padding_does_not_escape():
    """A partial last group is completed with a word that fits: 9 fitting
    words make two groups and no outlier."""
    w = np.full(9, 0x3F80, np.uint16)
    h = nf12.header(nf12.encode(w))
    assert h["n_groups"] == 2 and h["n_escaped"] == 0
    w[8] = 0x4000
    h = nf12.header(nf12.encode(w))
    assert h["n_escaped"] == 1


def test_escape_costs_28_bytes_per_group():
    """An escaped group keeps its 12-byte slot and adds 16 escape bytes; the
    other sections do not depend on the number of outliers."""
    n = 8 * 4096
    base = np.full(n, 0x3C00, np.uint16)
    h0 = nf12.header(nf12.encode(base))
    worse = base.copy()
    worse[::8 * 16] = 0      # one outlier every 16 groups: 256 outliers
    h1 = nf12.header(nf12.encode(worse))
    assert h1["n_escaped"] == 256 and h0["n_escaped"] == 0
    assert h1["off_escape"] == h0["off_escape"]
    assert h1["off_escape"] - h1["off_slots"] >= 12 * h1["n_groups"]
    assert h1["total_bytes"] - h0["total_bytes"] == 16 * 256


def test_gaussian_outlier_rate_and_size():
    """N(0, 0.02) weights: an element is an outlier when |w| < 2^-15 or
    |w| >= 2; a group escapes when any of its 8 elements is one.  The rate
    follows from the normal distribution; the size is near 12/16 of BF16
    (the page: roughly a quarter saved)."""
    n = 1 << 22
    w = W.normal_bf16((n,), seed=3)
    c = nf12.encode(w)
    h = nf12.header(c)
    # probability that rounding to BF16 gives |w| < 2^-15 (round to nearest:
    # below the midpoint between the largest word under 2^-15 and 2^-15)
    lim = (2.0 ** -15) * (1 - 2.0 ** -9)
    p = math.erf(lim / (0.02 * math.sqrt(2)))
    q = 1 - (1 - p) ** 8
    g = h["n_groups"]
    sd = math.sqrt(g * q * (1 - q))
    assert abs(h["n_escaped"] - g * q) < 5 * sd, (h["n_escaped"], g * q)
    # 12 slot bytes, 1/8 flag byte, 1/16 prefix byte and 16q escape bytes
    # per 16 bytes of BF16
    ratio = h["total_bytes"] / (2 * n)
    assert abs(ratio - (12 + 1 / 8 + 1 / 16 + 16 * q) / 16) < 0.001, ratio
    assert (nf12.decode(c, n) == w).all()


def test_check_rejects_inconsistent_containers():
    w = W.normal_bf16((8 * 300,), seed=5)
    w[::97] = 0
    c = nf12.encode(w)
    h = nf12.header(c)
    assert nf12.check(c) == 0 and h["n_escaped"] > 0

    def bad(mut):
        x = c.copy()
        mut(x)
        return nf12.check(x)

    assert bad(lambda x: x.__setitem__(0, ord("X"))) == nf12.E_FORMAT                       # magic
    assert bad(lambda x: x.__setitem__(8, 2)) == nf12.E_FORMAT                              # version
    assert bad(lambda x: x.__setitem__(32, x[32] + 1)) == nf12.E_FORMAT                      # n_escaped
    assert bad(lambda x: x.__setitem__(h["off_flags"], x[h["off_flags"]] ^ 1)) == nf12.E_FORMAT   # a flag
    assert bad(lambda x: x.__setitem__(h["off_prefix"] + 4, x[h["off_prefix"] + 4] + 1)) == nf12.E_FORMAT
    assert bad(lambda x: x.__setitem__(100, 1)) == nf12.E_FORMAT                            # reserved
    esc_group = int(np.flatnonzero(np.unpackbits(c[h["off_flags"]:h["off_flags"] + 8], bitorder="little"))[0])
    slot = h["off_slots"] + 12 * esc_group
    assert bad(lambda x: x.__setitem__(slot, 1)) == nf12.E_FORMAT                           # outlier slot
    assert nf12.check(c[:h["total_bytes"] - 1]) == nf12.E_FORMAT                            # truncated


# ---- the pins have teeth: a plausible mistake planted in a copy of the
#      oracle's C source makes at least one of them fail

MUTATIONS = [
    ("restores 0110 instead of 0111", "e = 0x70u | ((code >> 7) & 0xFu)", "e = 0x60u | ((code >> 7) & 0xFu)"),
    ("tests only three exponent bits", "return (exponent_of(w) >> 4) == 0x7u;", "return (exponent_of(w) >> 5) == 0x3u;"),
    ("sign one bit too high", "return (sign_of(w) << 11) |", "return (sign_of(w) << 12) |"),
    ("packs bits most significant first", "slot[(12 * i + b) / 8] |= (uint8_t)(1u << ((12 * i + b) % 8));",
     "slot[(12 * i + b) / 8] |= (uint8_t)(0x80u >> ((12 * i + b) % 8));"),
    ("completes the last group with zeros", "#define NF_PAD_WORD 0x3800u", "#define NF_PAD_WORD 0x0000u"),
    ("prefix counts the word's own outliers",
     "        if (g % 64 == 0) nput32(out + L.off_prefix + 4 * (g / 64), (uint32_t)e);\n        if (group_fits(w, n, g)) {",
     "        if (group_fits(w, n, g)) {\n            if (g % 64 == 63) nput32(out + L.off_prefix + 4 * (g / 64), (uint32_t)e);"),
]


def _battery() -> bool:
    try:
        for r in _rows("nf12_fields.txt"):
            word, fits, code = r.split()[:3]
            if nf12.fits(int(word, 16)) != (fits == "1"):
                return False
            if fits == "1" and nf12.code(int(word, 16)) != int(code, 16):
                return False
        for r in _rows("nf12_groups.txt"):
            left, right = r.split("|")
            words = np.array([int(x, 16) for x in left.split()], np.uint16)
            c = nf12.encode(words)
            h = nf12.header(c)
            if c[h["off_slots"]:h["off_slots"] + 12].tobytes() != bytes(int(x, 16) for x in right.split()):
                return False
        w = W.exhaustive_words()
        c = nf12.encode(w)
        if nf12.check(c) != 0 or not (nf12.decode(c, w.size) == w).all():
            return False
        rng = np.random.default_rng(1)
        for n in (9, 130, 600):
            x = rng.integers(0x3700, 0x4080, n).astype(np.uint16)
            if nf12.encode(x).tobytes() != tiny.nf12_encode_tiny([int(v) for v in x]):
                return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    import subprocess
    src = open(nf12._SRC).read()
    assert src.count(old) == 1, name
    d = tmp_path / "m"
    d.mkdir()
    (d / "nf12_oracle.c").write_text(src.replace(old, new))
    (d / "nf12_oracle.h").write_text(open(os.path.join(os.path.dirname(nf12._SRC), "nf12_oracle.h")).read())
    so = d / "libm.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-o", str(so), str(d / "nf12_oracle.c")])
    with nf12.use_library(str(so)):
        assert not _battery(), name
    assert _battery()
