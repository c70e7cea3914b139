"""GPU parity: the HIP decoder (through the C ABI) against the source words
and the CPU oracle, on containers written by the oracle's encoder.

Bit-exact is the only bar: decoding is defined to return every BF16 word
unchanged (mlx-dfloat project page, introduction and "Status")."""
import numpy as np
import pytest

import oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from exponent_mixes import ENTROPY_MIXES, entropy_mix_words, random_exponent_case
from gpu_util import empty_words, log, oracle_encode_many, to_device_u8, to_device_words

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _decode_one(words: np.ndarray, guard: int = 64):
    """Oracle-encode, decode on the GPU, return (host output, guard ok)."""
    torch = _torch()
    c = oracle.encode(words)
    plan = df11.Plan([c])
    dc = to_device_u8(c)
    buf, out = empty_words(words.size, guard=guard)
    df11.decode(plan, 0, dc, out)
    df11.check(plan)
    torch.cuda.synchronize()
    host = buf.cpu().numpy().view(np.uint16)
    ok_guard = (host[:guard] == 0x5A5A).all() and (host[guard + words.size:] == 0x5A5A).all()
    return host[guard:guard + words.size], ok_guard, c


EDGE_SIZES = [1, 2, 15, 63, 64, 65, 511, 512, 1000, 1023, 1024, 1025, 8191, 32767, 32768, 32769,
              65536, 3 * 32768 + 1000]


@pytest.mark.parametrize("n", EDGE_SIZES)
def test_edge_sizes_bit_exact(n):
    log(f"edge size n={n}")
    w = W.normal_bf16((n,), seed=1000 + n)
    got, guard, c = _decode_one(w)
    assert guard, "decoder wrote outside its output"
    assert (got == w).all()
    assert (got == oracle.decode(c, n)).all()


def test_exhaustive_65536_words():
    """Every exponent (8-bit codes) and every raw byte, incl. NaN payloads."""
    log("exhaustive 65536")
    w = W.exhaustive_words()
    got, guard, _ = _decode_one(w)
    assert guard and (got == w).all()


def test_shuffled_exhaustive_words():
    log("shuffled exhaustive")
    w = W.exhaustive_words()[np.random.default_rng(3).permutation(65536)]
    w = np.concatenate([w, w[::-1], w[:1234]])
    got, guard, _ = _decode_one(w)
    assert guard and (got == w).all()


def test_single_and_two_symbol_tensors():
    log("single / two symbols")
    w = ((np.arange(100000) % 256).astype(np.uint16) | np.uint16(127 << 7))
    got, guard, _ = _decode_one(w)
    assert guard and (got == w).all()
    w = np.where(np.arange(70001) % 5 == 0, 0x3F80, 0xC000).astype(np.uint16)
    got, guard, _ = _decode_one(w)
    assert guard and (got == w).all()


def test_long_codes_at_the_cap():
    """Fibonacci exponent counts (26 symbols, 317,810 words): the optimal code
    would be 25 deep, so the 24-bit cap binds and the longest codes take the
    kernel's canonical-limit path."""
    log("long codes")
    fib = [1, 1]
    while len(fib) < 26:
        fib.append(fib[-1] + fib[-2])
    exps = np.repeat(np.arange(90, 116, dtype=np.uint16), fib)
    exps = exps[np.random.default_rng(9).permutation(exps.size)]
    raw = np.random.default_rng(10).integers(0, 256, exps.size).astype(np.uint16)
    w = ((raw & 0x80) << 8) | (exps << 7) | (raw & 0x7F)
    c = oracle.encode(w)
    assert int(oracle.header(c)["code_len"].max()) == 24
    got, guard, _ = _decode_one(w)
    assert guard and (got == w).all()


def test_heavy_tail_slice():
    log("heavy tail slice")
    w = W.heavy_tail_bf16((1 << 20,), seed=5)
    got, guard, c = _decode_one(w)
    assert guard and (got == w).all()


def test_uniform_exponents_use_the_unstaged_path():
    """8-bit codes everywhere: the chunk's codes exceed the LDS staging area,
    so the kernel reads them straight from global memory."""
    log("unstaged path")
    w = np.random.default_rng(77).integers(0, 65536, 5 * 32768 + 17).astype(np.uint16)
    got, guard, _ = _decode_one(w)
    assert guard and (got == w).all()


def test_batched_mixed_sizes_one_call():
    torch = _torch()
    log("batched mixed sizes")
    sizes = [3072, 3072 * 3072 // 16, 1, 32768, 32769, 100003, 65536, 7]
    ws = [W.normal_bf16((n,), seed=i, std=0.02 if i % 2 else 0.05, mean=0.0 if i % 3 else 1.0)
          for i, n in enumerate(sizes)]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    bufs = [empty_words(n, guard=32) for n in sizes]
    df11.decode_batch(plan, dcs, [o for _, o in bufs])
    df11.check(plan)
    torch.cuda.synchronize()
    for w, (buf, _), n in zip(ws, bufs, sizes):
        host = buf.cpu().numpy().view(np.uint16)
        assert (host[32:32 + n] == w).all()
        assert (host[:32] == 0x5A5A).all() and (host[32 + n:] == 0x5A5A).all()


def test_tiles_reused_after_partial_chunks():
    """A workgroup decodes several chunks in turn into one LDS tile, which
    its assembly clears behind itself; a partial chunk's last windows run a
    few codes past the chunk's end, and those tile bytes are cleared
    separately.  Forty tensors of 20 whole chunks plus a partial one (every
    residue mod 8, a few near a store block's end), more chunks than the
    launch has workgroups, two launches in a row: every word exact."""
    torch = _torch()
    log("tiles reused after partial chunks")
    residues = [1, 2, 3, 4, 5, 6, 7, 8, 9, 13, 15, 17, 2047, 2049, 4095, 30001, 32767]
    sizes = [20 * 32768 + residues[i % len(residues)] for i in range(40)]
    mixes = list(ENTROPY_MIXES)
    ws = [W.normal_bf16((n,), seed=7000 + i) if i % 3 else entropy_mix_words(mixes[i % len(mixes)], n)
          for i, n in enumerate(sizes)]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    assert sum(i["n_chunks"] for i in plan.infos) > 768
    dcs = [to_device_u8(c) for c in cs]
    for rep in range(2):
        bufs = [empty_words(n, guard=16) for n in sizes]
        df11.decode_batch(plan, dcs, [o for _, o in bufs])
        df11.check(plan)
        torch.cuda.synchronize()
        for w, (buf, _), n in zip(ws, bufs, sizes):
            host = buf.cpu().numpy().view(np.uint16)
            assert (host[16:16 + n] == w).all(), (rep, n)
            assert (host[:16] == 0x5A5A).all() and (host[16 + n:] == 0x5A5A).all()


def test_more_tensors_than_one_launch():
    """70 tensors: the batch is split into launches of 64."""
    torch = _torch()
    log("70 tensors")
    ws = [W.normal_bf16((5000 + 37 * i,), seed=i) for i in range(70)]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    outs = [torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda") for w in ws]
    df11.decode_batch(plan, dcs, outs)
    df11.check(plan)
    for w, o in zip(ws, outs):
        assert (o.cpu().numpy().view(np.uint16) == w).all()


def test_non_default_stream_and_repeats():
    torch = _torch()
    log("non-default stream")
    w = W.normal_bf16((300000,), seed=42)
    c = oracle.encode(w)
    plan = df11.Plan([c])
    dc = to_device_u8(c)
    s = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(s):
        for _ in range(3):
            o = torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda")
            df11.decode(plan, 0, dc, o, stream=s)
            outs.append(o)
    df11.check(plan, stream=s)
    for o in outs:
        assert (o.cpu().numpy().view(np.uint16) == w).all()


def test_one_plan_from_four_host_threads():
    """Four host threads, each with a stream and outputs of its own, enqueue
    20 batched decodes of one plan at the same time (the library hands out
    the plan's ticket counters under a lock, and ctypes calls run without
    the interpreter lock); every output exact, the flag clear."""
    import threading
    torch = _torch()
    log("one plan, four host threads")
    sizes = [2 * 32768 + 11, 300001, 7]
    ws = [W.normal_bf16((n,), seed=80 + i) for i, n in enumerate(sizes)]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def run(t):
        try:
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for _ in range(20):
                    o = [torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda") for n in sizes]
                    df11.decode_batch(plan, dcs, o, stream=s)
                    outs.append(o)
            s.synchronize()
            results[t] = outs
        except Exception as e:  # reported by the main thread
            errors.append(e)

    th = [threading.Thread(target=run, args=(t,)) for t in range(4)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors, errors
    df11.check(plan)
    for outs in results:
        for o in outs:
            for w, oo in zip(ws, o):
                assert (oo.cpu().numpy().view(np.uint16) == w).all()


def test_ticket_counters_across_many_launches_and_streams():
    """Every launch takes its chunks from one of the plan's ticket counters,
    which its last workgroup clears.  160 launches (single and batched, on
    two streams that may run side by side); every output must be exact."""
    torch = _torch()
    log("ticket counters: 160 launches on two streams")
    sizes = [3 * 32768 + 5, 900001, 40000]
    ws = [W.normal_bf16((n,), seed=60 + i) for i, n in enumerate(sizes)]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for r in range(40):
        o = [torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda") for n in sizes]
        ob = [torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda") for n in sizes]
        s1.wait_stream(torch.cuda.current_stream())   # (the fills come first)
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            df11.decode(plan, 0, dcs[0], o[0], stream=s1)
            df11.decode(plan, 2, dcs[2], o[2], stream=s1)
        with torch.cuda.stream(s2):
            df11.decode(plan, 1, dcs[1], o[1], stream=s2)
            df11.decode_batch(plan, dcs, ob, stream=s2)
        outs += [o, ob]
    df11.check(plan, stream=s1)
    df11.check(plan, stream=s2)
    torch.cuda.synchronize()
    for o in outs:
        for w, t in zip(ws, o):
            assert (t.cpu().numpy().view(np.uint16) == w).all()


def test_more_queued_launches_than_ticket_counters():
    """A launch gets a ticket counter only once the last launch on it has
    finished (its last workgroup reports to the host).  300 decodes of one
    plan are queued on a stream held back behind a long copy on another
    stream (more than the plan's 256 counters, so the host waits for
    counters to come free), with 200 more on two free streams meanwhile; the
    held-back launches then run beside later ones.  Every output is exact and
    the flag stays clear."""
    torch = _torch()
    log("300 held-back launches and 200 free ones")
    n = 1600 * 32768 + 999          # more chunks than workgroups: tickets are taken
    w = W.normal_bf16((n,), seed=77)
    c = oracle_encode_many([w])[0]
    plan = df11.Plan([c])
    dc = to_device_u8(c)
    held, s1, s2, cp = (torch.cuda.Stream() for _ in range(4))
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big2 = torch.empty_like(big)
    outs = [torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    with torch.cuda.stream(cp):
        for _ in range(6):
            big2.copy_(big)
        ev = torch.cuda.Event()
        ev.record(cp)
    held.wait_event(ev)
    for i in range(300):
        df11.decode(plan, 0, dc, outs[0], stream=held)
    for i in range(100):
        df11.decode(plan, 0, dc, outs[1], stream=s1)
        df11.decode(plan, 0, dc, outs[2], stream=s2)
    for st in (held, s1, s2):
        df11.check(plan, stream=st)
    torch.cuda.synchronize()
    for o in outs:
        assert (o.cpu().numpy().view(np.uint16) == w).all()


def test_corrupted_stream_sets_the_flag():
    """A flipped bit in the device copy of the stream: the kernel keeps every
    access in bounds, and df11_check reports the inconsistency (or the words
    differ, when the flip swaps two codes of equal length)."""
    torch = _torch()
    log("corrupted stream")
    w = W.normal_bf16((200000,), seed=8)
    c = oracle.encode(w)
    h = oracle.header(c)
    plan = df11.Plan([c])
    bad = c.copy()
    bad[h["off_stream"] + 4000] ^= 0x40
    dc = to_device_u8(bad)
    o = torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda")
    df11.decode(plan, 0, dc, o)
    try:
        df11.check(plan)
        flagged = False
    except df11.DF11Error as e:
        flagged = e.status == 5
    differs = not (o.cpu().numpy().view(np.uint16) == w).all()
    assert flagged or differs
    # the flag is cleared by the check; a clean decode passes again
    df11.decode(plan, 0, to_device_u8(c), o)
    df11.check(plan)
    assert (o.cpu().numpy().view(np.uint16) == w).all()


@pytest.mark.parametrize("window", [1, 200, 300, 511])
def test_wrong_window_gap_sets_the_flag(window):
    """The gap of one window of chunk 1 raised by one bit in the device copy:
    the window before it decodes exactly and ends where that window's first
    code really starts, one bit before the index says, so df11_check must
    report DF11_E_CORRUPT; the kernel writes only inside the output (guard
    words stay) and the other chunks decode exactly."""
    torch = _torch()
    log(f"wrong window gap, window {window}")
    w = W.normal_bf16((3 * 32768 + 77,), seed=9)
    c = oracle.encode(w)
    h = oracle.header(c)
    plan = df11.Plan([c])
    bad = c.copy()
    off = h["off_windows"] + 2 * (512 + window)
    ent = int(bad[off:off + 2].view(np.uint16)[0])
    assert ent & 0x7FF and (ent >> 11) < 24
    bad[off:off + 2] = np.array([ent + (1 << 11)], np.uint16).view(np.uint8)
    buf, o = empty_words(w.size, guard=64)
    df11.decode(plan, 0, to_device_u8(bad), o)
    with pytest.raises(df11.DF11Error) as e:
        df11.check(plan)
    assert e.value.status == 5
    host = buf.cpu().numpy().view(np.uint16)
    assert (host[:64] == 0x5A5A).all() and (host[64 + w.size:] == 0x5A5A).all()
    assert (host[64:64 + 32768] == w[:32768]).all()
    assert (host[64 + 65536:64 + w.size] == w[65536:]).all()
    df11.decode(plan, 0, to_device_u8(c), o)
    df11.check(plan)
    assert (o.cpu().numpy().view(np.uint16) == w).all()


@pytest.mark.parametrize("r,n", [(0.0603, 32768 * 64), (0.09, 32768 * 16 + 32000)])
def test_chunks_ending_near_the_source_end(r, n):
    """Six exponents at probability q and four at r (3- and 4-bit codes, 3 +
    4r bits per element).  At r = 0.0603 (3.24 bits) many chunks' codes end
    within a few hundred bits of the 13 KiB LDS staging area's end; at r =
    0.09 (3.36 bits) the codes are read from global memory and the last
    chunk ends at the stream's end.  Windows there start within 24 bits per
    counted look-up of the end of what the decoder's peeks may read: each
    still starts where its index says, and the tensor decodes exactly, in a
    batch and on its own."""
    torch = _torch()
    log(f"chunks ending near the source end r={r}")
    q = (1 - 4 * r) / 6
    w = W.exponent_mix_bf16(n, seed=41, probs=[q] * 6 + [r] * 4)
    small = W.normal_bf16((5000,), seed=42)
    cs = oracle_encode_many([w, small])
    h = oracle.header(cs[0])
    ci = cs[0][h["off_chunk_index"]:h["off_chunk_index"] + 16 * (h["n_chunks"] + 1)].view(np.uint64)
    bits = np.diff(ci[0::2].astype(np.int64))
    if r < 0.07:
        assert ((bits > 105900) & (bits < 106240)).sum() >= 8   # staged, near the cap
    else:
        assert bits[-1] > 3.3 * 32000                           # not staged
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    bufs = [empty_words(m, guard=32) for m in (n, 5000)]
    df11.decode_batch(plan, dcs, [o for _, o in bufs])
    df11.check(plan)
    for src, (buf, _), m in zip([w, small], bufs, (n, 5000)):
        host = buf.cpu().numpy().view(np.uint16)
        assert (host[32:32 + m] == src).all()
    buf, out = empty_words(n, guard=32)
    df11.decode(plan, 0, dcs[0], out)
    df11.check(plan)
    host = buf.cpu().numpy().view(np.uint16)
    assert (host[32:32 + n] == w).all()
    assert (host[:32] == 0x5A5A).all() and (host[32 + n:] == 0x5A5A).all()


@pytest.mark.parametrize("order", ["short_first", "long_first"])
def test_chunks_sorted_by_code_length(order):
    """Each chunk's words sorted by code length: one exponent at probability
    1/2 (a 1-bit code) and the other 255 uniform (8- and 9-bit codes), so
    that the windows over the short codes hold hundreds of codes and those
    over the long ones a few dozen. The wave minimum that bounds the counted
    look-ups is small, most look-ups run masked, and the waves differ
    widely in work."""
    log(f"chunks sorted by code length, {order}")
    w = W.exponent_mix_bf16(32768 * 12 + 999, seed=5, probs=[255.0] + [1.0] * 255, e0=0)
    code_len = oracle.header(oracle.encode(w))["code_len"].astype(np.int64)
    for c0 in range(0, w.size, 32768):
        part = w[c0:c0 + 32768]
        key = code_len[(part >> 7) & 0xFF]
        idx = np.argsort(key if order == "short_first" else -key, kind="stable")
        w[c0:c0 + 32768] = part[idx]
    got, ok_guard, c = _decode_one(w, guard=32)
    h = oracle.header(c)
    win = c[h["off_windows"]:h["off_windows"] + 1024 * h["n_chunks"]].view(np.uint16) & 0x7FF
    assert win.max() >= 250 and win[win > 0].min() <= 40   # the skew is there
    assert ok_guard
    assert (got == w).all()


@pytest.mark.parametrize("name", list(ENTROPY_MIXES))
def test_exponent_entropy_sweep(name):
    """Code rates from 1 to 7.7 bits per element (exponents drawn from a given
    distribution, random sign and fraction), so that chunk code sizes fall on
    both sides of the LDS staging area and anywhere relative to the ends of
    what the decoder reads; 40 whole chunks and a ragged one, bit-exact."""
    log(f"entropy sweep {name}")
    w = entropy_mix_words(name, 32768 * 40 + 3001)
    got, ok_guard, _ = _decode_one(w, guard=32)
    assert ok_guard
    assert (got == w).all()


def test_source_hash_verifies_decoded_output():
    """Hashed containers (the oracle's, flag DF11_FLAG_SHA256) decode like
    plain ones; the decoded device words verify against the header's hash
    with no source at hand; a flipped fraction bit in the device copy, which
    no structural check can see, fails the verify."""
    torch = _torch()
    log("source hash verify")
    ws = [W.normal_bf16((65536 + 77,), seed=21), W.heavy_tail_bf16((40000,), seed=22)]
    cs = [oracle.encode(w, sha256=True) for w in ws]
    plan = df11.Plan(cs)
    outs = [torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda") for w in ws]
    df11.decode_batch(plan, [to_device_u8(c) for c in cs], outs)
    df11.check(plan)
    for w, c, o in zip(ws, cs, outs):
        assert (o.cpu().numpy().view(np.uint16) == w).all()
        assert df11.verify_decoded(c, o)
    bad = cs[0].copy()
    bad[oracle.header(bad)["off_raw"] + 999] ^= 0x01
    df11.decode(plan, 0, to_device_u8(bad), outs[0])
    df11.check(plan)                       # the structure is intact
    assert not df11.verify_decoded(cs[0], outs[0])


def test_bad_arguments_are_rejected():
    torch = _torch()
    w = W.normal_bf16((1000,), seed=2)
    c = oracle.encode(w)
    plan = df11.Plan([c])
    dc = to_device_u8(c)
    o = torch.full((w.size + 8,), 0x5A5A, dtype=torch.int16, device="cuda")
    with pytest.raises(df11.DF11Error) as e:
        df11.decode(plan, 0, dc, o[1:])      # misaligned output
    assert e.value.status == 1
    with pytest.raises(df11.DF11Error):
        df11.decode(plan, 1, dc, o)          # no tensor 1
    with pytest.raises(df11.DF11Error):
        df11.Plan([c[:100]])                 # truncated metadata
    # what the binding checks before the call (the library cannot see the
    # size of a device buffer): nothing is enqueued for these
    with pytest.raises(ValueError):
        df11.decode(plan, 0, dc, o[:w.size - 8])                 # output too small
    with pytest.raises(ValueError):
        df11.decode(plan, 0, dc[:-16], o)                        # container too short
    with pytest.raises(ValueError):
        df11.decode(plan, 0, dc, o.view(torch.int32))            # not 16-bit words
    with pytest.raises(ValueError):
        df11.decode(plan, 0, dc, o.cpu())                        # not on the GPU
    with pytest.raises(ValueError):
        df11.decode_batch(plan, [dc], [o.reshape(-1, 8)[:, :4]])  # not contiguous
    df11.decode(plan, 0, dc, o[:w.size])
    df11.check(plan)
    assert (o[:w.size].cpu().numpy().view(np.uint16) == w).all()


def _sampled_oracle_chunks(c, words, n_samples=3):
    """Compare a few chunks with the oracle's own chunk decode."""
    h = oracle.header(c)
    rng = np.random.default_rng(h["n_chunks"])
    for ch in sorted(set(rng.integers(0, h["n_chunks"], n_samples).tolist()) | {h["n_chunks"] - 1}):
        lo, hi = ch * 32768, min(h["n_elems"], (ch + 1) * 32768)
        assert (oracle.decode_chunk(c, ch, hi - lo) == words[lo:hi]).all()


def _full_workload(specs):
    torch = _torch()
    ws = [s.make().reshape(-1) for s in specs]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    srcs = [to_device_words(w) for w in ws]
    outs = [torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda") for w in ws]
    df11.decode_batch(plan, dcs, outs)
    df11.check(plan)
    torch.cuda.synchronize()
    for s, o in zip(srcs, outs):
        assert torch.equal(s, o)
    return ws, cs


def test_workload_single_2048():
    log("workload single_2048")
    ws, cs = _full_workload(W.single_2048())
    _sampled_oracle_chunks(cs[0], ws[0])


def test_workload_llama8b_block():
    log("workload llama8b_block")
    ws, cs = _full_workload(W.llama8b_block())
    _sampled_oracle_chunks(cs[4], ws[4])


def test_workload_heavy_tail_8192():
    log("workload heavy_tail_8192")
    ws, cs = _full_workload(W.heavy_tail_8192())
    assert int(oracle.header(cs[0])["code_len"].max()) == 24
    _sampled_oracle_chunks(cs[0], ws[0])


def test_workload_flux_dit_block():
    log("workload flux_dit_block")
    ws, cs = _full_workload(W.flux_dit_block())
    _sampled_oracle_chunks(cs[-1], ws[-1])
    _sampled_oracle_chunks(cs[12], ws[12])


def test_bw_control_moves_every_byte():
    """The bandwidth control reads the source and writes every output unit."""
    torch = _torch()
    src = torch.full((3 * 4096 + 16,), 1, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(5 * 4096 + 32, dtype=torch.uint8, device="cuda")
    df11.bw_control(src, dst)
    torch.cuda.synchronize()
    words = dst.view(torch.int32).reshape(-1, 4).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    assert (words[:, 1:] == 0x01010101).all()
    assert (words[:, 0] == (0x01010101 ^ np.arange(words.shape[0]))).all()
    with pytest.raises(df11.DF11Error):
        df11.bw_control(src[:15], dst)                # size not a multiple of 16
    with pytest.raises(df11.DF11Error):
        df11.bw_control(src, src)                     # overlapping regions
    with pytest.raises(df11.DF11Error):
        df11.bw_control(dst, src)                     # source above the output: not all of it would be read


def test_decode_batch_replays_from_a_hip_graph():
    """decode_batch captured into a HIP graph (three launches, each with its
    own ticket counter slot), replayed five times with eager work and
    synchronization in between; every replay must give exact words, so every
    launch's last workgroup must have cleared its counter."""
    torch = _torch()
    log("hip graph replays")
    sizes = [32768 * 3 + 11, 250000, 4096]
    ws = [W.normal_bf16((n,), seed=200 + i) for i, n in enumerate(sizes)]
    cs = oracle_encode_many(ws)
    plan = df11.Plan(cs)
    dcs = [to_device_u8(c) for c in cs]
    outs = [[torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda") for n in sizes] for _ in range(3)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())               # (the fills come first)
    with torch.cuda.stream(s):
        df11.decode_batch(plan, dcs, outs[0], stream=s)      # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for o in outs:
            df11.decode_batch(plan, dcs, o, stream=s)
    for rep in range(5):
        for o in outs:
            for t in o:
                t.fill_(rep + 1)                               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            for w, t in zip(ws, o):
                assert (t.cpu().numpy().view(np.uint16) == w).all(), rep
    df11.check(plan)


def test_random_distributions_in_one_batched_launch():
    """60 seeded random cases (sizes up to 200,000 words, random exponent
    sets and probabilities, Fibonacci counts that reach the 24-bit cap, an
    empty tensor possible) in the oracle's containers, decoded by one
    batched launch (60 tensors, 60 code tables): every output equals its
    source words, with guard words on both sides untouched; and one batched
    GPU encoder call over the same words writes the oracle's bytes."""
    import torch
    log("random distributions, batched")
    ws = [random_exponent_case(seed, 200_000) for seed in range(60)]
    conts = oracle_encode_many(ws)
    assert max(int(oracle.header(c)["code_len"].max()) for c, w in zip(conts, ws) if w.size) == 24
    plan = df11.Plan(conts)
    d_conts = [to_device_u8(c) for c in conts]
    bufs = [empty_words(w.size, guard=16) for w in ws]
    df11.decode_batch(plan, d_conts, [o for _, o in bufs])
    df11.check(plan)
    torch.cuda.synchronize()
    for seed, (w, (buf, out)) in enumerate(zip(ws, bufs)):
        got = buf.cpu().numpy().view(np.uint16)
        assert (got[16:16 + w.size] == w).all(), seed
        assert (got[:16] == 0x5A5A).all() and (got[16 + w.size:] == 0x5A5A).all(), seed
    log("random distributions, GPU encoder")
    ts = [torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to("cuda") for w in ws]
    gs = df11.encode_device_batch(ts)
    torch.cuda.synchronize()
    for seed, (g, c) in enumerate(zip(gs, conts)):
        assert g.numel() == c.size and (g.cpu().numpy() == c).all(), seed
