"""The oracle's SHA-256 and the optional source hash in the container header.

The df11pack page ("Beyond the official format") describes a per-tensor
SHA-256 in the header so that a verify finds corruption without the source,
the tensor bytes unchanged.  The oracle's SHA-256 is written from FIPS 180-4
(constants derived from the primes' roots); it is pinned here to Python's
hashlib, an independent implementation, on messages around every padding
boundary."""
import hashlib

import numpy as np
import pytest

import oracle
from lossless_bf16_weight_amd import workloads as W


@pytest.mark.parametrize("n", [0, 1, 3, 55, 56, 57, 63, 64, 65, 111, 112, 119, 120, 127, 128, 129, 1000, 100003])
def test_sha256_matches_hashlib(n):
    b = np.random.default_rng(n).integers(0, 256, n).astype(np.uint8).tobytes()
    assert oracle.sha256(b) == hashlib.sha256(b).digest()


def test_sha256_on_the_standard_messages():
    for m in (b"abc", b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq", b"a" * 1000):
        assert oracle.sha256(m) == hashlib.sha256(m).digest()


def _source_digest(w):
    return hashlib.sha256(np.ascontiguousarray(w, dtype="<u2").tobytes()).digest()


def test_hashed_container_holds_the_source_digest_and_nothing_else_changes():
    w = W.normal_bf16((70000,), seed=4)
    plain = oracle.encode(w)
    hashed = oracle.encode(w, sha256=True)
    h = oracle.header(hashed)
    assert h["flags"] == oracle.FLAG_SHA256 and h["sha256"] == _source_digest(w)
    assert oracle.header(plain)["flags"] == 0 and oracle.header(plain)["sha256"] == bytes(32)
    # every other byte is the same: the flag word and the digest differ only
    diff = np.flatnonzero(plain != hashed)
    assert plain.size == hashed.size and ((diff == 12) | ((diff >= 176) & (diff < 208))).all()
    assert oracle.check(hashed) == 0 and (oracle.decode(hashed, w.size) == w).all()


def test_hash_catches_what_the_structure_cannot():
    w = W.normal_bf16((40000,), seed=5)
    c = oracle.encode(w, sha256=True)
    h = oracle.header(c)
    bad = c.copy()
    bad[h["off_raw"] + 1234] ^= 0x01            # a fraction bit: every structure check passes
    assert oracle.check(c) == 0
    plain = oracle.encode(w)
    plain_bad = plain.copy()
    plain_bad[h["off_raw"] + 1234] ^= 0x01
    assert oracle.check(plain_bad) == 0          # without the hash the change is invisible
    assert oracle.check(bad) == oracle.E_CORRUPT
    bad = c.copy()
    bad[190] ^= 0x80                             # the stored digest itself
    assert oracle.check(bad) == oracle.E_CORRUPT
    bad = plain.copy()
    bad[200] = 1                                 # digest bytes without the flag
    assert oracle.check(bad) == oracle.E_FORMAT
    bad = c.copy()
    bad[12] |= 2                                 # an undefined flag bit
    assert oracle.check(bad) == oracle.E_FORMAT


def test_empty_and_single_word_tensors_hash():
    for w in (np.zeros(0, np.uint16), np.array([0x3F80], np.uint16)):
        c = oracle.encode(w, sha256=True)
        assert oracle.header(c)["sha256"] == _source_digest(w) and oracle.check(c) == 0
