"""The product library's SHA-256 and its source-hash option (no GPU).

df11_sha256 is pinned to Python's hashlib (an independent implementation) at
every padding boundary; df11_encode_ex with DF11_FLAG_SHA256 must write the
oracle's hashed container byte for byte; df11_validate reports the hash and
rejects hash bytes without the flag; df11_verify_words follows the df11pack
page's verify outcomes (pass, a check failed, could not check)."""
import hashlib

import numpy as np
import pytest

import oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W


@pytest.mark.parametrize("n", [0, 1, 55, 56, 63, 64, 65, 119, 120, 128, 4097, 1000003])
def test_sha256_matches_hashlib(n):
    b = np.random.default_rng(n).integers(0, 256, n).astype(np.uint8)
    assert df11.sha256(b) == hashlib.sha256(b.tobytes()).digest()


def test_portable_sha256_matches_hashlib():
    """The portable code path (the library picks the processor's SHA
    extensions when it has them; the environment variable forces the
    portable one), in a fresh process."""
    import os
    import subprocess
    import sys
    code = ("import hashlib, numpy as np, lossless_bf16_weight_amd as d\n"
            "for n in (0, 1, 55, 56, 63, 64, 65, 119, 120, 128, 100003):\n"
            "    b = np.random.default_rng(n).integers(0, 256, n).astype(np.uint8)\n"
            "    assert d.sha256(b) == hashlib.sha256(b.tobytes()).digest(), n\n"
            "print('ok')\n")
    env = dict(os.environ, DF11_SHA256_PORTABLE="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-2000:]


@pytest.mark.parametrize("n", [0, 1, 1000, 32768, 32769, 100003])
def test_hashed_encode_matches_oracle_bytes(n):
    w = W.normal_bf16((n,), seed=n)
    want = oracle.encode(w, sha256=True)
    for t in (1, 4):
        got = df11.encode(w, threads=t, sha256=True)
        assert got.size == want.size and (got == want).all()
    # the unhashed container differs in the flag word and the digest only
    plain = df11.encode(w)
    diff = np.flatnonzero(plain != want)
    assert ((diff >= 12) & (diff < 16) | (diff >= 176) & (diff < 208)).all()


def test_validate_reports_and_checks_the_hash_fields():
    w = W.normal_bf16((5000,), seed=3)
    c = df11.encode(w, sha256=True)
    info = df11.validate(c)
    assert info["flags"] == df11.FLAG_SHA256
    assert info["sha256"] == hashlib.sha256(w.astype("<u2").tobytes()).digest()
    assert df11.validate(df11.encode(w))["sha256"] == bytes(32)
    plain = df11.encode(w)
    bad = plain.copy()
    bad[190] = 7                                            # digest bytes without the flag
    assert df11.validate_status(bad) == df11._lib.E_FORMAT
    bad = c.copy()
    bad[12] |= 4                                            # an undefined flag bit
    assert df11.validate_status(bad) == df11._lib.E_UNSUPPORTED


def test_verify_words_outcomes():
    w = W.normal_bf16((40000,), seed=6)
    c = df11.encode(w, sha256=True)
    assert df11.verify(c, w)
    assert df11.verify(c[:df11.validate(c)["meta_bytes"]], w)     # the metadata prefix is enough
    bad = w.copy()
    bad[31337] ^= 1
    assert not df11.verify(c, bad)
    assert df11.verify_status(c, bad) == df11._lib.E_CORRUPT
    assert df11.verify_status(df11.encode(w), w) == df11._lib.E_UNSUPPORTED   # no hash to check
    assert df11.verify_status(c, w[:-1]) == df11._lib.E_ARG
    with pytest.raises(df11.DF11Error):
        df11.verify(df11.encode(w), w)
