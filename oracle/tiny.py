"""Pure-Python helpers for brute-force checks of the oracle on tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as the rest of `oracle/`).

Nothing here calls the C oracle: these are independent, deliberately naive
routines that the tests hold the oracle against:

* `brute_force_min_cost`: the minimum of sum(f*l) over ALL length vectors with
  Kraft sum <= 1 and lengths <= cap (exhaustive; alphabets <= 8).
* `heap_huffman_cost`: the textbook Huffman procedure (repeatedly join the two
  lightest weights); its cost is the optimum without a length cap.
* `canonical_code_strings`: canonical code values by the counting
  construction of RFC 1951 section 3.2.2 (bl_count / next_code), as strings.
* `decode_with_strings`: decodes a version-4 container by matching code
  strings against the bit string of the stream, ignoring every index.
* `nf12_encode_tiny`: an NF12 container built a second way (field values by
  slicing the 16-bit pattern as a string, each group as one 96-bit integer).
"""
from __future__ import annotations

import heapq
import itertools
import struct


def brute_force_min_cost(freq, cap):
    """Exhaustive optimum of sum(f*l) subject to sum(2^-l) <= 1, 1 <= l <= cap."""
    syms = [s for s, f in enumerate(freq) if f > 0]
    if not syms:
        return 0
    if len(syms) == 1:
        return freq[syms[0]] * 1
    best = None
    for ls in itertools.product(range(1, cap + 1), repeat=len(syms)):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            cost = sum(freq[s] * l for s, l in zip(syms, ls))
            if best is None or cost < best:
                best = cost
    return best


def heap_huffman_cost(freq):
    """Textbook Huffman: cost = sum of the weights of all internal nodes."""
    ws = [f for f in freq if f > 0]
    if len(ws) <= 1:
        return sum(ws)
    heapq.heapify(ws)
    cost = 0
    while len(ws) > 1:
        a = heapq.heappop(ws)
        b = heapq.heappop(ws)
        cost += a + b
        heapq.heappush(ws, a + b)
    return cost


def heap_huffman_depth(freq):
    """Depth of the textbook Huffman tree (ties broken by insertion order)."""
    items = [(f, i, 0) for i, f in enumerate(freq) if f > 0]
    if len(items) <= 1:
        return len(items)
    heapq.heapify(items)
    k = len(freq)
    while len(items) > 1:
        fa, _, da = heapq.heappop(items)
        fb, _, db = heapq.heappop(items)
        heapq.heappush(items, (fa + fb, k, max(da, db) + 1))
        k += 1
    return items[0][2]


def canonical_code_strings(lengths):
    """RFC 1951 3.2.2 counting construction; returns {symbol: bit string}."""
    max_bits = max(lengths) if len(lengths) else 0
    bl_count = [0] * (max_bits + 2)
    for l in lengths:
        if l:
            bl_count[l] += 1
    next_code = [0] * (max_bits + 2)
    code = 0
    for bits in range(1, max_bits + 1):
        code = (code + bl_count[bits - 1]) << 1
        next_code[bits] = code
    out = {}
    for s in range(len(lengths)):
        l = lengths[s]
        if l:
            out[s] = format(next_code[l], "0%db" % l)
            next_code[l] += 1
    return out


def _u64(b, o):
    return struct.unpack_from("<Q", b, o)[0]


def decode_with_strings(container: bytes):
    """Decode a version-4 container through its code strings only."""
    b = bytes(container)
    assert b[:8] == b"DF11HIPC"
    n = _u64(b, 16)
    total_bits = _u64(b, 104)
    off_stream = _u64(b, 136)
    off_raw = _u64(b, 152)
    lengths = list(b[208:464])
    table = {v: s for s, v in canonical_code_strings(lengths).items()}
    nbytes = (total_bits + 7) // 8
    bits = "".join(format(x, "08b") for x in b[off_stream:off_stream + nbytes])[:total_bits]
    out = []
    cur = ""
    for ch in bits:
        cur += ch
        if cur in table:
            out.append(table[cur])
            cur = ""
    assert cur == "" and len(out) == n
    words = []
    for j, e in enumerate(out):
        r = b[off_raw + j]
        words.append(((r & 0x80) << 8) | (e << 7) | (r & 0x7F))
    return words


def nf12_encode_tiny(words):
    """Byte string of the NF12 container of `words` (a list of ints)."""
    n = len(words)
    padded = list(words) + [0x3800] * (-n % 8)
    groups = [padded[i:i + 8] for i in range(0, len(padded), 8)]
    G = len(groups)
    n_words = (G + 63) // 64

    def fits(w):
        return format(w, "016b")[1:5] == "0111"

    def code(w):
        s = format(w, "016b")
        return int(s[0] + s[5:9] + s[9:16], 2)

    esc = [g for g in range(G) if not all(fits(w) for w in groups[g])]
    align = lambda x: (x + 255) // 256 * 256
    off_slots = 256
    off_flags = align(off_slots + 12 * G)
    off_prefix = align(off_flags + 8 * n_words)
    off_escape = align(off_prefix + 4 * n_words)
    total = align(off_escape + 16 * len(esc))
    out = bytearray(total)
    out[0:8] = b"NF12HIPC"
    struct.pack_into("<II", out, 8, 1, 0)
    struct.pack_into("<QQQQQQQQ", out, 16, n, G, len(esc), off_slots, off_flags, off_prefix, off_escape, total)
    for g in range(G):
        if g in esc:
            continue
        v = sum(code(w) << (12 * i) for i, w in enumerate(groups[g]))
        out[off_slots + 12 * g:off_slots + 12 * g + 12] = v.to_bytes(12, "little")
    for w in range(n_words):
        flags = sum(1 << (g - 64 * w) for g in esc if 64 * w <= g < 64 * (w + 1))
        struct.pack_into("<Q", out, off_flags + 8 * w, flags)
        struct.pack_into("<I", out, off_prefix + 4 * w, sum(1 for g in esc if g < 64 * w))
    for k, g in enumerate(esc):
        struct.pack_into("<8H", out, off_escape + 16 * k, *groups[g])
    return bytes(out)
