"""Helpers shared by the GPU parity tests (test-side only)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def oracle_encode_many(arrays):
    """Oracle containers for many tensors, one tensor per worker thread (the
    oracle itself stays single-threaded per tensor)."""
    import oracle
    with ThreadPoolExecutor(threads()) as ex:
        return list(ex.map(oracle.encode, arrays))


def to_device_u8(c: np.ndarray):
    import torch
    t = torch.empty(c.size, dtype=torch.uint8, device="cuda")
    t.copy_(torch.from_numpy(np.ascontiguousarray(c)))
    return t


def to_device_words(w: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(w).reshape(-1).view(np.int16)).to("cuda")


def empty_words(n: int, guard: int = 0, fill: int = 0x5A5A):
    """Output buffer of n 16-bit words with `guard` canary words on each side
    (the slice handed to the decoder stays 16-byte aligned)."""
    import torch
    assert guard % 8 == 0
    buf = torch.full((n + 2 * guard,), fill - 65536 if fill >= 32768 else fill,
                     dtype=torch.int16, device="cuda")
    return buf, buf[guard:guard + n]


def _mix(r):
    """Six exponents at probability q and four at r: 3- and 4-bit codes,
    3 + 4r bits per element."""
    q = (1 - 4 * r) / 6
    return [q] * 6 + [r] * 4


# exponent distributions from 1 to 7.7 bits per element (by their code rate)
ENTROPY_MIXES = {
    "1bit": [1, 1], "1.5bit": [2, 1, 1], "2bit": [1] * 4, "2.4bit": [1] * 5, "3bit": [1] * 8,
    "3.2bit": _mix(0.05), "3.24bit": _mix(0.0603), "3.28bit": _mix(0.07), "3.36bit": _mix(0.09),
    "3.35bit": _mix(0.12), "3.7bit": [1] * 12, "4bit": [1] * 16, "5bit": [1] * 32, "6bit": [1] * 64,
    "7bit": [1] * 128, "7.7bit": [1] * 200,
}


def entropy_mix_words(name: str, n: int):
    """n words with the exponent distribution ENTROPY_MIXES[name], centred on
    exponent 127, random sign and fraction."""
    from lossless_bf16_weight_amd import workloads as W
    probs = ENTROPY_MIXES[name]
    return W.exponent_mix_bf16(n, seed=len(probs) * 7 + 3, probs=probs, e0=max(1, 127 - len(probs) // 2))
