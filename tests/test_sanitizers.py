"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host code (container validation, which parses untrusted
headers and indexes; the encoders; SHA-256; the NF12 host code) and the C
oracles are built with -fsanitize=address,undefined into two small drivers
(tests/sanitize/), which then run over a corpus written here: valid
containers and word files, and a few thousand containers broken on purpose
(header fields, code lengths, chunk and window index entries, random byte
flips, truncations).  Every validation must return a status without a
sanitizer report, every word file must round-trip, and the sanitized encoder
must write the bytes the normal build writes.  The host side of the
decode's ticket-counter slots is checked in the same driver (a slot is not
given out again before the device reports its launch finished, and a
captured launch keeps its slot), and so are the decode tables: every look-up
the kernel's arithmetic makes on them (first level, subtables, canonical
limits) gives the codes the canonical code has, on random streams for 400
codes."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from exponent_mixes import entropy_mix_words

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_bf16_weight_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    if not (os.path.exists(CLANG) and shutil.which("gcc")):
        pytest.skip("clang++ or gcc not available")
    d = tmp_path_factory.mktemp("asan")
    host = str(d / "host_asan")
    r = subprocess.run([CLANG, "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                        os.path.join(SAN, "host_driver.cpp")] +
                       [os.path.join(CSRC, f) for f in ("host.cpp", "encode.cpp", "nf12.cpp", "sha256.cpp")] +
                       ["-o", host, "-L/opt/rocm/lib", "-lamdhip64", "-lpthread", "-Wl,-rpath,/opt/rocm/lib"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    orc = str(d / "oracle_asan")
    r = subprocess.run(["gcc", "-std=c99", *FLAGS, "-I" + os.path.join(ROOT, "oracle"),
                        os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "df11_oracle.c"),
                        os.path.join(ROOT, "oracle", "nf12_oracle.c"), "-o", orc],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return host, orc


def _word_sets():
    rng = np.random.default_rng(7)
    return {
        "normal": W.normal_bf16((100003,), seed=1),
        "every_word": W.exhaustive_words(),
        "heavy": W.heavy_tail_bf16((3 * 32768 + 5,), seed=2),
        "one_symbol": np.full(70000, 0x3F80, np.uint16),
        "two_words": np.array([0x3F80, 0xC000], np.uint16),
        "one": np.array([0x7FC1], np.uint16),
        "empty": np.zeros(0, np.uint16),
        "mix": entropy_mix_words(sorted(__import__("exponent_mixes").ENTROPY_MIXES)[3], 2 * 32768 + 77),
        "random": rng.integers(0, 65536, 40000, dtype=np.uint16),
    }


def _broken_df11(c, rng, n_random):
    """Containers broken on purpose: every header field, code lengths, index
    entries, random flips in the metadata prefix and anywhere, truncations."""
    out = []
    h = oracle.header(c)
    meta = int(df11.validate(c)["meta_bytes"])
    for off, size in [(0, 8), (8, 4), (12, 4), (16, 8), (24, 4), (28, 4), (32, 8), (96, 1), (98, 2),
                      (100, 4), (104, 8), (112, 8), (120, 8), (136, 8), (144, 8), (152, 8), (160, 8), (168, 8)]:
        for val in (0, 1, 2 ** (8 * size) - 1, 2 ** (8 * size - 1), int(rng.integers(0, 2 ** 31))):
            b = c.copy()
            b[off:off + size] = np.frombuffer(int(val % 2 ** (8 * size)).to_bytes(size, "little"), np.uint8)
            out.append(b)
    for s in range(0, 256, 17):
        for v in (0, 1, 24, 25, 31, 255):
            b = c.copy()
            b[208 + s] = v
            out.append(b)
    if h["n_chunks"]:
        off_ci, off_win = int(h["off_chunk_index"]), int(h["off_windows"])
        for k in range(min(4, h["n_chunks"] + 1)):
            for v in (0, 1, 2 ** 63, 2 ** 64 - 1, int(h["total_bits"]) + 1):
                b = c.copy()
                b[off_ci + 16 * k:off_ci + 16 * k + 8] = np.frombuffer(int(v).to_bytes(8, "little"), np.uint8)
                out.append(b)
        for k in (0, 1, 255, 511):
            for v in (0, 1, 0x07FF, 0xF800, 0xFFFF):
                b = c.copy()
                b[off_win + 2 * k:off_win + 2 * k + 2] = np.frombuffer(int(v).to_bytes(2, "little"), np.uint8)
                out.append(b)
    for _ in range(n_random):
        b = c.copy()
        hi = meta if rng.random() < 0.8 else c.size
        for _ in range(int(rng.integers(1, 9))):
            b[int(rng.integers(0, hi))] ^= np.uint8(1 << int(rng.integers(0, 8)))
        out.append(b)
    for cut in (1, 16, 4096, c.size // 2):
        if cut < c.size:
            out.append(c[: c.size - cut].copy())
    return out


def _broken_nf12(c, rng, n_random):
    out = []
    for off, size in [(0, 8), (8, 4), (12, 4), (16, 8), (24, 8), (32, 8), (40, 8), (48, 8), (56, 8), (64, 8),
                      (72, 8)]:
        for val in (0, 1, 2 ** (8 * size) - 1, int(rng.integers(0, 2 ** 31))):
            b = c.copy()
            b[off:off + size] = np.frombuffer(int(val % 2 ** (8 * size)).to_bytes(size, "little"), np.uint8)
            out.append(b)
    for _ in range(n_random):
        b = c.copy()
        for _ in range(int(rng.integers(1, 9))):
            b[int(rng.integers(0, c.size))] ^= np.uint8(1 << int(rng.integers(0, 8)))
        out.append(b)
    for cut in (1, 16, c.size // 2):
        if cut < c.size:
            out.append(c[: c.size - cut].copy())
    return out


def _run(exe, manifest):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, manifest], capture_output=True, text=True, timeout=900, env=env)
    report = r.stderr
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], report[-6000:])
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-6000:]
    return r.stdout


def test_host_code_and_oracle_under_sanitizers(drivers, tmp_path):
    host, orc = drivers
    rng = np.random.default_rng(2024)
    lines = ["slots -", "luts -"]
    words = _word_sets()
    for name, w in words.items():
        p = tmp_path / f"{name}.u16"
        w.astype("<u2").tofile(p)
        lines.append(f"words {p}")
    n_df11 = 0
    for name in ("normal", "every_word", "heavy", "one_symbol", "one", "empty"):
        c = df11.encode(words[name])
        for k, b in enumerate([c] + _broken_df11(c, rng, 400)):
            p = tmp_path / f"{name}.{k}.df11"
            b.tofile(p)
            lines.append(f"df11 {p}")
            n_df11 += 1
    for name in ("normal", "every_word", "one"):
        c = df11.nf12_encode(words[name])
        for k, b in enumerate([c] + _broken_nf12(c, rng, 200)):
            p = tmp_path / f"{name}.{k}.nf12"
            b.tofile(p)
            lines.append(f"nf12 {p}")
    manifest = tmp_path / "manifest.txt"
    manifest.write_text("\n".join(lines) + "\n")
    assert n_df11 > 2000

    out = _run(host, str(manifest))
    assert out.startswith("ok:"), out
    # the sanitized encoder wrote the normal build's bytes
    for name, w in words.items():
        got = np.fromfile(tmp_path / f"{name}.u16.asan.df11", np.uint8)
        assert (got == df11.encode(w)).all() and got.size == df11.encode(w).size, name
    out = _run(orc, str(manifest))
    assert out.startswith("ok:"), out
