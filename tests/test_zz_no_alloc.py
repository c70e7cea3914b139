"""The GPU encoder's entry point that allocates nothing
(df11_encode_device_batch_noalloc), called through the C ABI: its containers
must be those df11_encode_device_batch writes, byte for byte, on calls in a
row whose inputs shrink (the fixed histogram array keeps the previous call's
counts, so a call that did not clear it would build another code), from
several host threads at once, and into output buffers full of garbage; more
than 64 tensors is refused before anything runs."""
import threading

import numpy as np
import pytest

import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from exponent_mixes import ENTROPY_MIXES, entropy_mix_words
from gpu_util import log

pytestmark = pytest.mark.gpu


def _dev(ws):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to("cuda") for w in ws]


def _garbage_outs(ts, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randint(0, 256, (df11.container_bound(t.numel()),), dtype=torch.uint8, device="cuda", generator=g)
            for t in ts]


def _same(got, want, what):
    import torch
    torch.cuda.synchronize()
    assert len(got) == len(want), what
    for k, (g, w) in enumerate(zip(got, want)):
        g, w = g.cpu().numpy(), w.cpu().numpy()
        assert g.size == w.size and (g == w).all(), (what, k)


def test_noalloc_matches_the_allocating_entry_point_on_shrinking_calls():
    import torch
    mixes = sorted(ENTROPY_MIXES)
    first = [W.normal_bf16((3 * 32768 + 77,), seed=11), W.heavy_tail_bf16((200003,), seed=12),
             W.exhaustive_words(), entropy_mix_words(mixes[-1], 5 * 32768 + 1001), np.zeros(0, np.uint16),
             W.normal_bf16((1_500_000,), seed=13)]
    # smaller, fewer, other exponent statistics: any count left from the
    # first call would change these tensors' codes
    second = [entropy_mix_words(mixes[0], 32768 + 5), np.full(1, 0x3F80, np.uint16)]
    for step, ws in enumerate((first, second)):
        log(f"no-alloc encode call {step}: {len(ws)} tensors, {sum(w.size for w in ws)} words")
        ts = _dev(ws)
        want = df11.encode_device_batch(ts)
        got = df11.encode_device_batch(ts, outs=_garbage_outs(ts, step), noalloc=True)
        _same(got, want, f"call {step}")
        for w, g in zip(ws, got):   # and the host encoder's bytes
            h = df11.encode(w)
            assert g.numel() == h.size and (g.cpu().numpy() == h).all()
    # a third call on another stream, back to the first inputs
    s = torch.cuda.Stream()
    ts = _dev(first[:3])
    want = df11.encode_device_batch(ts)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        got = df11.encode_device_batch(ts, stream=s, noalloc=True)
    s.synchronize()
    _same(got, want, "other stream")


def test_noalloc_from_several_host_threads():
    """Four threads, three calls each, on streams of their own: the library
    makes the calls take turns on the one histogram array."""
    import torch
    jobs = [[W.normal_bf16((32768 * (1 + t) + 3 * c,), seed=100 + 10 * t + c),
             W.heavy_tail_bf16((40000 + 7 * t,), seed=200 + 10 * t + c)] for t in range(4) for c in range(3)]
    want = [df11.encode_device_batch(_dev(ws)) for ws in jobs]
    torch.cuda.synchronize()
    got = [None] * len(jobs)
    errors = []

    def run(t):
        try:
            s = torch.cuda.Stream()
            for c in range(3):
                k = 3 * t + c
                ts = _dev(jobs[k])
                with torch.cuda.stream(s):
                    got[k] = df11.encode_device_batch(ts, stream=s, noalloc=True)
            s.synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    log("no-alloc encode from 4 threads")
    th = [threading.Thread(target=run, args=(t,)) for t in range(4)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors, errors
    for k in range(len(jobs)):
        _same(got[k], want[k], f"job {k}")


def test_noalloc_tensor_limit():
    log("no-alloc encode: 64 tensors, then 65")
    ws = [W.normal_bf16((100 + 37 * k,), seed=k) for k in range(65)]
    ts = _dev(ws)
    _same(df11.encode_device_batch(ts[:64], noalloc=True), df11.encode_device_batch(ts[:64]), "64 tensors")
    with pytest.raises(df11.DF11Error) as e:
        df11.encode_device_batch(ts, noalloc=True)
    assert e.value.status == 3   # DF11_E_UNSUPPORTED
    assert "at most 64" in str(e.value)
