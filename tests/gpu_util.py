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

