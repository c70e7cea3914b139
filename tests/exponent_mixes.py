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
