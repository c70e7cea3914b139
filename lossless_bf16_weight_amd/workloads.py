"""Seeded synthetic BF16 workloads.

This module holds only input generation (random numbers, a float32 -> BF16
round-to-nearest-even cast and tensor shapes).  It contains none of the
compression arithmetic, imports nothing else from this package, and is the one
module that both the decoder's tests/benchmark and the oracle's tests draw
their inputs from.

Recipe (the same for every tensor):
  * a tensor with seed `s` is generated in blocks of 2**20 elements; block `b`
    draws from ``numpy.random.default_rng([s, b])`` (PCG64), so blocks can be
    generated in parallel and the result does not depend on the thread count;
  * samples are drawn in float64, scaled (and shifted), cast to float32, then
    rounded to BF16 with round-to-nearest-even on the float32 bit pattern,
    ``(u + 0x7FFF + ((u >> 16) & 1)) >> 16`` -- the rounding torch's
    ``.to(torch.bfloat16)`` performs (df11pack page, "Models": sources are cast
    with torch; compressr page, dtype cast with round-to-nearest-even);
  * "N(mu, sigma)" means mean mu and standard deviation sigma.

Workloads (sizes from the LLM / DiT shapes they stand in for):
  * ``single_2048``: one 2048x2048 tensor, N(0, 0.02), seed 0;
  * ``llama8b_block``: q/o 4096x4096, k/v 1024x4096, gate/up 14336x4096,
    down 4096x14336, N(0, 0.02), seeds 0..6 in that order;
  * ``heavy_tail_8192``: one 8192x8192 tensor: Student-t(nu=3) x 0.01; one
    permutation (seed 0) picks disjoint index sets: 1% exact +0.0, then 0.1%
    outliers (a fresh t(3) x 0.01 draw, x 1000 before rounding), then 0.01%
    subnormals (sign and a
    fraction in 1..127 drawn at random, exponent 0);
  * ``flux_dit_block``: 8x 3072x3072, 2x 12288x3072, 2x 3072x12288,
    6x 3072x18432 with N(0, 0.02), then 16 vectors of 3072 with N(1, 0.05);
    seeds 0..33 in that order;
  * ``llama8b_stack``: 32 blocks of the ``llama8b_block`` layout, tensor t of
    layer l with seed 7*l + t (layer 0 is ``llama8b_block``), plus a
    128256x4096 embedding, N(0, 0.02), seed 224.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, List, Optional, Tuple

import numpy as np

BLOCK = 1 << 20


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _blocked(n: int, seed: int, fill: Callable[[np.random.Generator, int], np.ndarray],
             threads: Optional[int] = None) -> np.ndarray:
    out = np.empty(n, np.uint16)
    nblk = (n + BLOCK - 1) // BLOCK

    def work(b):
        lo = b * BLOCK
        hi = min(n, lo + BLOCK)
        rng = np.random.default_rng([seed, b])
        out[lo:hi] = bf16_rne(fill(rng, hi - lo).astype(np.float32))

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(work, range(nblk)))
    return out


def normal_bf16(shape, seed: int, std: float = 0.02, mean: float = 0.0,
                threads: Optional[int] = None) -> np.ndarray:
    n = int(np.prod(shape))
    w = _blocked(n, seed, lambda rng, m: rng.standard_normal(m) * std + mean, threads)
    return w.reshape(shape)


def heavy_tail_bf16(shape, seed: int = 0, threads: Optional[int] = None) -> np.ndarray:
    n = int(np.prod(shape))
    scale = 0.01
    base = _blocked(n, seed, lambda rng, m: rng.standard_t(3, m) * scale, threads)
    rng = np.random.default_rng([seed, 0x5EED])
    perm = rng.permutation(n)
    n_zero, n_out, n_sub = round(n * 0.01), round(n * 0.001), round(n * 0.0001)
    zero_idx = perm[:n_zero]
    out_idx = perm[n_zero:n_zero + n_out]
    sub_idx = perm[n_zero + n_out:n_zero + n_out + n_sub]
    base[zero_idx] = 0
    # outliers: a fresh t(3) x 0.01 sample, multiplied by 1000 before rounding
    t = rng.standard_t(3, n_out) * scale * 1000.0
    base[out_idx] = bf16_rne(t.astype(np.float32))
    sign = rng.integers(0, 2, n_sub).astype(np.uint16) << np.uint16(15)
    frac = rng.integers(1, 128, n_sub).astype(np.uint16)
    base[sub_idx] = sign | frac
    return base.reshape(shape)


def exponent_mix_bf16(n: int, seed: int, probs, e0: int = 120) -> np.ndarray:
    """n BF16 words whose biased exponent is e0 + k with probability probs[k],
    with a random sign and 7-bit fraction: a tensor whose coded size per
    element is set directly by the exponent distribution."""
    rng = np.random.default_rng(seed)
    p = np.asarray(probs, np.float64)
    e = e0 + rng.choice(len(p), size=n, p=p / p.sum())
    sign = rng.integers(0, 2, n)
    frac = rng.integers(0, 128, n)
    return ((sign << 15) | (e << 7) | frac).astype(np.uint16)


@dataclass
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    seed: int
    kind: str = "normal"      # normal | heavy_tail
    mean: float = 0.0
    std: float = 0.02

    @property
    def numel(self) -> int:
        return int(np.prod(self.shape))

    def make(self, threads: Optional[int] = None) -> np.ndarray:
        if self.kind == "heavy_tail":
            return heavy_tail_bf16(self.shape, self.seed, threads)
        return normal_bf16(self.shape, self.seed, self.std, self.mean, threads)


LLAMA_BLOCK = [
    ("q_proj", (4096, 4096)), ("k_proj", (1024, 4096)), ("v_proj", (1024, 4096)),
    ("o_proj", (4096, 4096)), ("gate_proj", (14336, 4096)), ("up_proj", (14336, 4096)),
    ("down_proj", (4096, 14336)),
]


def single_2048() -> List[TensorSpec]:
    return [TensorSpec("w", (2048, 2048), 0)]


def llama8b_block(layer: int = 0) -> List[TensorSpec]:
    return [TensorSpec(f"layers.{layer}.{n}", s, 7 * layer + t)
            for t, (n, s) in enumerate(LLAMA_BLOCK)]


def heavy_tail_8192() -> List[TensorSpec]:
    return [TensorSpec("w", (8192, 8192), 0, kind="heavy_tail")]


def flux_dit_block() -> List[TensorSpec]:
    shapes = ([(3072, 3072)] * 8 + [(12288, 3072)] * 2 + [(3072, 12288)] * 2
              + [(3072, 18432)] * 6)
    specs = [TensorSpec(f"mat{i}", s, i) for i, s in enumerate(shapes)]
    specs += [TensorSpec(f"vec{i}", (3072,), len(shapes) + i, mean=1.0, std=0.05)
              for i in range(16)]
    return specs


def llama8b_stack_layers(n_layers: int = 32) -> List[List[TensorSpec]]:
    """Per-layer tensor lists; the embedding is its own last group."""
    groups = [llama8b_block(l) for l in range(n_layers)]
    groups.append([TensorSpec("embed_tokens", (128256, 4096), 224)])
    return groups


WORKLOADS = {
    "single_2048": single_2048,
    "llama8b_block": llama8b_block,
    "heavy_tail_8192": heavy_tail_8192,
    "flux_dit_block": flux_dit_block,
}


def exhaustive_words() -> np.ndarray:
    """Every one of the 65,536 BF16 bit patterns once, in order."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)
