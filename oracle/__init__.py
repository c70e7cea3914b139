"""Oracle for DFloat11-style lossless BF16 weight compression.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline timing may import this package; the product library
(`lossless_bf16_weight_amd`) never imports it, and this package never imports
the product.

The arithmetic lives in plain C (`df11_oracle.c`, one thread, bit-serial
decoding); this module only marshals numpy arrays through ctypes.  `tiny.py`
holds a second, pure-Python encoder/decoder for brute-force checks on tiny
inputs.

Sources: mlx-dfloat project page, introduction and its 16-bit weight diagram
(exponent replaced by a variable-length code, sign + fraction kept as one raw
byte, decoded output identical bit for bit); df11pack project page, "Use"
(verify: structure, sampled chunks, full decode).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "df11_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, E_ARG, E_FORMAT, E_CORRUPT, E_TRUNCATED = 0, 1, 2, 3, 4
FLAG_SHA256 = 1
CHUNK = 32768
WINDOWS = 512
CAP = 24


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
             "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _configure(L):
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.oracle_code_lengths.argtypes = [u64p, ctypes.c_int, u8p]
    L.oracle_canonical_codes.argtypes = [u8p, u32p]
    L.oracle_container_bound.argtypes = [ctypes.c_uint64]
    L.oracle_container_bound.restype = ctypes.c_uint64
    L.oracle_encode.argtypes = [u16p, ctypes.c_uint64, ctypes.c_int, u64p, u8p,
                                ctypes.c_uint64, u64p]
    L.oracle_encode_flags.argtypes = [u16p, ctypes.c_uint64, ctypes.c_int, u64p, ctypes.c_uint32, u8p,
                                      ctypes.c_uint64, u64p]
    L.oracle_sha256.argtypes = [u8p, ctypes.c_uint64, u8p]
    L.oracle_decode.argtypes = [u8p, ctypes.c_uint64, u16p, ctypes.c_uint64]
    L.oracle_decode_chunk.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint64, u16p]
    L.oracle_decode_window.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                     u16p, u64p, u64p]
    L.oracle_check.argtypes = [u8p, ctypes.c_uint64]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Run the oracle's Python API against another build of df11_oracle.c
    (used by the tests that plant mistakes in a copy of the oracle)."""
    global _lib
    saved = lib()
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def code_lengths(freq, cap: int = CAP) -> np.ndarray:
    f = np.ascontiguousarray(freq, dtype=np.uint64)
    assert f.shape == (256,)
    out = np.zeros(256, np.uint8)
    st = lib().oracle_code_lengths(_p(f, ctypes.c_uint64), cap, _p(out, ctypes.c_uint8))
    if st:
        raise OracleError(st, "code_lengths")
    return out


def canonical_codes(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(256, np.uint32)
    lib().oracle_canonical_codes(_p(ln, ctypes.c_uint8), _p(out, ctypes.c_uint32))
    return out


def sha256(data) -> bytes:
    """SHA-256 digest of a bytes-like object (FIPS 180-4, the oracle's C)."""
    b = np.frombuffer(bytes(data), dtype=np.uint8) if not isinstance(data, np.ndarray) else \
        np.ascontiguousarray(data).view(np.uint8).reshape(-1)
    out = np.zeros(32, np.uint8)
    src = b if b.size else np.zeros(1, np.uint8)
    lib().oracle_sha256(_p(src, ctypes.c_uint8), b.size, _p(out, ctypes.c_uint8))
    return out.tobytes()


def encode(words: np.ndarray, shape=None, sha256: bool = False) -> np.ndarray:
    """Encode a uint16 array (BF16 bit patterns) into a version-4 container;
    with sha256, the header holds the SHA-256 of the source words."""
    w = np.ascontiguousarray(words, dtype=np.uint16).reshape(-1)
    shape = tuple(words.shape) if shape is None else tuple(shape)
    dims = np.array(shape if shape else (0,), dtype=np.uint64)
    ndim = len(shape)
    cap = int(lib().oracle_container_bound(w.size))
    out = np.zeros(cap, np.uint8)
    nbytes = np.zeros(1, np.uint64)
    st = lib().oracle_encode_flags(_p(w, ctypes.c_uint16), w.size, ndim, _p(dims, ctypes.c_uint64),
                                   FLAG_SHA256 if sha256 else 0,
                                   _p(out, ctypes.c_uint8), cap, _p(nbytes, ctypes.c_uint64))
    if st:
        raise OracleError(st, "encode")
    return out[: int(nbytes[0])].copy()


def decode(container: np.ndarray, n: int) -> np.ndarray:
    c = np.ascontiguousarray(container, dtype=np.uint8)
    out = np.zeros(n, np.uint16)
    st = lib().oracle_decode(_p(c, ctypes.c_uint8), c.size, _p(out, ctypes.c_uint16), n)
    if st:
        raise OracleError(st, "decode")
    return out


def decode_chunk(container: np.ndarray, chunk: int, n_chunk: int) -> np.ndarray:
    c = np.ascontiguousarray(container, dtype=np.uint8)
    out = np.zeros(n_chunk, np.uint16)
    st = lib().oracle_decode_chunk(_p(c, ctypes.c_uint8), c.size, chunk,
                                   _p(out, ctypes.c_uint16))
    if st:
        raise OracleError(st, "decode_chunk")
    return out


def decode_window(container: np.ndarray, chunk: int, win: int):
    """Decode one window of a chunk; returns (words, end_bit)."""
    c = np.ascontiguousarray(container, dtype=np.uint8)
    out = np.zeros(CHUNK, np.uint16)
    n_out = np.zeros(1, np.uint64)
    end = np.zeros(1, np.uint64)
    st = lib().oracle_decode_window(_p(c, ctypes.c_uint8), c.size, chunk, win,
                                  _p(out, ctypes.c_uint16), _p(n_out, ctypes.c_uint64),
                                  _p(end, ctypes.c_uint64))
    if st:
        raise OracleError(st, "decode_window")
    return out[: int(n_out[0])].copy(), int(end[0])


def check(container: np.ndarray) -> int:
    """Structural check; returns the oracle status (0 = valid)."""
    c = np.ascontiguousarray(container, dtype=np.uint8)
    return int(lib().oracle_check(_p(c, ctypes.c_uint8), c.size))


# ---- header fields of a version-4 container (layout in df11_oracle.c) ----

def header(container: np.ndarray) -> dict:
    c = np.ascontiguousarray(container, dtype=np.uint8)

    def u32(o):
        return int(c[o:o + 4].view(np.uint32)[0])

    def u16(o):
        return int(c[o:o + 2].view(np.uint16)[0])

    def u64(o):
        return int(c[o:o + 8].view(np.uint64)[0])

    ndim = u32(24)
    return {
        "n_elems": u64(16), "ndim": ndim,
        "dims": [u64(32 + 8 * i) for i in range(ndim)],
        "chunk_elems": u32(28), "max_code_len": int(c[96]), "windows": u16(98),
        "n_chunks": u32(100), "total_bits": u64(104),
        "off_chunk_index": u64(112), "off_windows": u64(120),
        "off_stream": u64(136), "stream_bytes": u64(144), "off_raw": u64(152),
        "raw_bytes": u64(160), "total_bytes": u64(168),
        "code_len": c[208:464].copy(),
        "flags": u32(12), "sha256": c[176:208].tobytes(),
    }
