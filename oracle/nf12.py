"""Oracle for NF12, the fixed-rate lossless BF16 format.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the arithmetic is
plain C (`nf12_oracle.c`, one element and one bit at a time); this module only
marshals numpy arrays through ctypes.

Source: the nf12 news page ("Developer open-sources nf12: lossless 12-bit
compression for BF16 models"), "How it works" and "Implementation details".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nf12_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnf12oracle.so")

OK, E_ARG, E_FORMAT = 0, 1, 2
HEADER = 256
PAD_WORD = 0x3800


def build(force: bool = True) -> str:
    """Compile nf12_oracle.c with gcc into oracle/libnf12oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u8p, u16p, u64p = (ctypes.POINTER(t) for t in (ctypes.c_uint8, ctypes.c_uint16, ctypes.c_uint64))
        L.oracle_nf12_fits.argtypes = [ctypes.c_uint16]
        L.oracle_nf12_code.argtypes = [ctypes.c_uint16]
        L.oracle_nf12_code.restype = ctypes.c_uint32
        L.oracle_nf12_word.argtypes = [ctypes.c_uint32]
        L.oracle_nf12_word.restype = ctypes.c_uint16
        L.oracle_nf12_bound.argtypes = [ctypes.c_uint64]
        L.oracle_nf12_bound.restype = ctypes.c_uint64
        L.oracle_nf12_encode.argtypes = [u16p, ctypes.c_uint64, u8p, ctypes.c_uint64, u64p]
        L.oracle_nf12_check.argtypes = [u8p, ctypes.c_uint64]
        L.oracle_nf12_decode.argtypes = [u8p, ctypes.c_uint64, u16p, ctypes.c_uint64]
        _lib = L
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def fits(word: int) -> bool:
    return bool(lib().oracle_nf12_fits(word))


def code(word: int) -> int:
    return int(lib().oracle_nf12_code(word))


def word(code: int) -> int:
    return int(lib().oracle_nf12_word(code))


def encode(words: np.ndarray) -> np.ndarray:
    """NF12 container (uint8 array) of a uint16 array of BF16 bit patterns."""
    w = np.ascontiguousarray(np.asarray(words).view(np.uint16).reshape(-1))
    cap = int(lib().oracle_nf12_bound(w.size))
    out = np.empty(cap, np.uint8)
    nbytes = ctypes.c_uint64(0)
    st = lib().oracle_nf12_encode(_p(w, ctypes.c_uint16), w.size, _p(out, ctypes.c_uint8), cap,
                                  ctypes.byref(nbytes))
    if st:
        raise RuntimeError(f"nf12 encode: oracle status {st}")
    return out[: nbytes.value].copy()


def check(container: np.ndarray) -> int:
    c = np.ascontiguousarray(container, dtype=np.uint8)
    return int(lib().oracle_nf12_check(_p(c, ctypes.c_uint8), c.size))


def decode(container: np.ndarray, n: int) -> np.ndarray:
    c = np.ascontiguousarray(container, dtype=np.uint8)
    out = np.zeros(n, np.uint16)
    st = lib().oracle_nf12_decode(_p(c, ctypes.c_uint8), c.size, _p(out, ctypes.c_uint16), n)
    if st:
        raise RuntimeError(f"nf12 decode: oracle status {st}")
    return out


def header(c: np.ndarray) -> dict:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    u64 = lambda o: int(c[o:o + 8].view(np.uint64)[0])
    return {"version": int(c[8:12].view(np.uint32)[0]), "n_elems": u64(16), "n_groups": u64(24),
            "n_escaped": u64(32), "off_slots": u64(40), "off_flags": u64(48), "off_prefix": u64(56),
            "off_escape": u64(64), "total_bytes": u64(72)}


import contextlib  # noqa: E402


@contextlib.contextmanager
def use_library(path: str):
    """Run this module's API against another build of nf12_oracle.c (used by
    the test that plants mistakes in a copy of the oracle)."""
    global _lib
    saved = lib()
    _lib = None
    real = _LIB_PATH
    try:
        globals()["_LIB_PATH"] = path
        lib()
        yield
    finally:
        globals()["_LIB_PATH"] = real
        _lib = saved
