"""Exponent distributions for parity sweeps over code rates: seeded inputs
only (the distributions and the words drawn from them), shared by the CPU
and GPU tests."""


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


def random_exponent_case(seed: int, max_n: int):
    """One seeded random case: a size in [0, max_n] (every tenth case a whole
    number of chunks, plus or minus a little) and a random set of 1 to 256
    exponents with Dirichlet-drawn probabilities (concentration from 0.05,
    very skewed, to 2); or, one case in four, exponents with Fibonacci
    counts (1, 1, 2, 3, 5, ...: the most skewed code tree, 25 of them reach
    the 24-bit length cap) in random order.  Sign and fraction bits
    uniform.  Returns the 16-bit words."""
    import numpy as np
    rng = np.random.default_rng([0xD11, seed])
    k = int(rng.integers(1, 257))
    syms = rng.choice(256, size=k, replace=False)
    if seed % 4 == 3:
        fib = [1, 1]
        while len(fib) < min(k, 25) and sum(fib) + fib[-1] + fib[-2] <= max_n:
            fib.append(fib[-1] + fib[-2])
        fib = fib[:k]
        e = np.repeat(syms[:len(fib)], fib).astype(np.uint16)
        e = e[rng.permutation(e.size)]
        n = e.size
    else:
        if seed % 10 == 0:
            n = int(32768 * rng.integers(1, max(2, max_n // 32768 + 1)) + rng.integers(-3, 4))
            n = max(0, min(n, max_n))
        else:
            n = int(rng.integers(0, max_n + 1))
        p = rng.dirichlet(np.full(k, float(rng.uniform(0.05, 2.0))))
        e = syms[rng.choice(k, size=n, p=p / p.sum())].astype(np.uint16)
    low = rng.integers(0, 256, size=n, dtype=np.uint16)
    return ((low & 0x80) << 8) | (e << 7) | (low & 0x7F)
