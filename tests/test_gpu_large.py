"""GPU parity at the largest size the tests reach: one tensor of
2^31 + 12,345 BF16 weights (65,537 chunks, about 5.6 G code bits), so that
element offsets pass 2^31 and stream bit offsets pass 2^32 (the container
format allows up to 2^46 elements and 2^24 chunks per tensor).

Checks: the GPU encoder's container equals the host encoder's byte for
byte; the whole output equals the source words (compared on the GPU); the
chunks on either side of element 2^31, the first and the last equal the
oracle's own chunk decode of the same container; guard words on both sides
of the output stay untouched; the same tensor decoded again in one batched
launch beside a small tensor gives the same words.

Input: 8 Mi Gaussian weights (sigma 0.02, as the Llama-8B block's tensors)
repeated, each repetition r with its fraction bits XORed with r mod 128, so
that the raw bytes differ from one repetition to the next (the exponent
statistics, and so the code, are those of the 8 Mi weights)."""
import numpy as np
import pytest

import oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from gpu_util import empty_words, log, threads, to_device_u8, to_device_words

pytestmark = pytest.mark.gpu

N_BIG = (1 << 31) + 12345
GUARD = 64
CANARY = 0x5A5A


def _big_words() -> np.ndarray:
    base = W.normal_bf16((1 << 23,), seed=41)
    w = np.empty(N_BIG, np.uint16)
    full = N_BIG // base.size
    reps = w[: full * base.size].reshape(full, base.size)
    reps[:] = base[None, :]
    reps ^= (np.arange(full, dtype=np.uint16) & 0x7F)[:, None]
    rest = N_BIG - full * base.size
    w[full * base.size:] = base[:rest] ^ np.uint16(full & 0x7F)
    return w


def _guards_intact(buf, n):
    import torch
    g = buf[:GUARD], buf[GUARD + n:]
    return all(bool((x == CANARY).all().item()) for x in g) and all(x.numel() == GUARD for x in g)


def test_tensor_past_2_31_elements_and_2_32_code_bits():
    import torch
    log(f"large tensor: {N_BIG} words, generating")
    w = _big_words()
    c = df11.encode(w, threads=threads())
    h = oracle.header(c)
    assert h["n_chunks"] == 65537 and h["total_bits"] > (1 << 32)
    # the oracle's chunk decodes of the same container
    last = h["n_chunks"] - 1
    for ch in (0, (1 << 31) // 32768 - 1, (1 << 31) // 32768, last - 1, last):
        lo, hi = ch * 32768, min(N_BIG, (ch + 1) * 32768)
        assert (oracle.decode_chunk(c, ch, hi - lo) == w[lo:hi]).all(), ch
    log(f"large tensor: container {c.size} bytes, {h['total_bits']} code bits; decoding")

    plan = df11.Plan([c])
    dc = to_device_u8(c)
    src = to_device_words(w)
    del w
    # the GPU encoder on the same words: the same bytes
    log("large tensor: GPU encoder")
    g = df11.encode_device(src)
    torch.cuda.synchronize()
    assert g.numel() == c.size and torch.equal(g, dc)
    del g
    buf, out = empty_words(N_BIG, guard=GUARD, fill=CANARY)
    df11.decode(plan, 0, dc, out)
    df11.check(plan)
    torch.cuda.synchronize()
    assert torch.equal(out, src)
    assert _guards_intact(buf, N_BIG)

    # again, batched with a small tensor in the same launch
    log("large tensor: batched with a small tensor")
    small = W.normal_bf16((3 * 32768 + 5,), seed=42)
    plan2 = df11.Plan([c, df11.encode(small)])
    ds = to_device_u8(df11.encode(small))
    buf.fill_(CANARY)
    sbuf, sout = empty_words(small.size, guard=GUARD, fill=CANARY)
    df11.decode_batch(plan2, [dc, ds], [out, sout])
    df11.check(plan2)
    torch.cuda.synchronize()
    assert torch.equal(out, src)
    assert torch.equal(sout, to_device_words(small))
    assert _guards_intact(buf, N_BIG) and _guards_intact(sbuf, small.size)
