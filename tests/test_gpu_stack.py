"""GPU parity of the just-in-time layer loop over a resident compressed stack:
32 Llama-3-8B-shaped blocks (7 tensors each, tensor t of layer l seeded
7*l + t) plus a 128256x4096 embedding, 7.5 G BF16 weights in all.  Every
container stays in HBM; each layer is decoded in turn, with one batched call,
into one reused BF16 buffer (mlx-dfloat project page, introduction: the
weights stay compressed in memory and each block is decoded on the GPU as it
runs).

Checks:
  * every tensor of every layer: SHA-256 of the decoded words equals the
    SHA-256 of the source words;
  * every tensor: two sampled chunks (and the last) equal the oracle's own
    chunk decode; layer 0: the oracle's full decode has the same SHA-256, and
    the product encoder's containers are byte-identical to the oracle's;
  * a timed pass over all 33 layers reports the sustained decode rate."""
import hashlib
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from gpu_util import log, threads, to_device_u8

pytestmark = pytest.mark.gpu


def _sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def _sampled_oracle_chunks(c, words, seed):
    h = oracle.header(c)
    rng = np.random.default_rng(seed)
    picks = set(rng.integers(0, h["n_chunks"], 2).tolist()) | {h["n_chunks"] - 1}
    for ch in sorted(picks):
        lo, hi = ch * 32768, min(h["n_elems"], (ch + 1) * 32768)
        assert (oracle.decode_chunk(c, ch, hi - lo) == words[lo:hi]).all(), (seed, ch)


def test_llama8b_stack_jit_layer_loop():
    import torch

    groups = W.llama8b_stack_layers(32)
    pool = ThreadPoolExecutor(threads())

    # ---- compress every layer and keep the containers resident in HBM
    t0 = time.time()
    plans, dconts, shas, counts = [], [], [], []
    for gi, g in enumerate(groups):
        ws = [s.make().reshape(-1) for s in g]
        cs = [df11.encode(w, shape=s.shape) for w, s in zip(ws, g)]
        shas.append(list(pool.map(_sha, ws)))
        counts.append([w.size for w in ws])
        list(pool.map(lambda a: _sampled_oracle_chunks(*a),
                      [(c, w, s.seed) for c, w, s in zip(cs, ws, g)]))
        if gi == 0:
            # the oracle's own containers and full decode of layer 0
            ocs = list(pool.map(oracle.encode, [w.reshape(s.shape) for w, s in zip(ws, g)]))
            for a, b in zip(cs, ocs):
                assert a.size == b.size and (a == b).all()
            full = list(pool.map(lambda a: _sha(oracle.decode(a[0], a[1])),
                                 [(c, w.size) for c, w in zip(cs, ws)]))
            assert full == shas[0]
        plans.append(df11.Plan(cs))
        dconts.append([to_device_u8(c) for c in cs])
        if gi % 8 == 0 or gi == len(groups) - 1:
            log(f"stack: layer group {gi} resident ({time.time() - t0:.1f} s)")
        del ws, cs
    resident = sum(int(c.numel()) for dc in dconts for c in dc)
    n_total = sum(sum(c) for c in counts)
    assert n_total == 32 * 218103808 + 128256 * 4096

    # ---- one reused output buffer, large enough for the largest group
    buf = torch.full((max(sum(c) for c in counts),), 0x5A5A, dtype=torch.int16, device="cuda")

    def views(ci):
        out, off = [], 0
        for n in ci:
            out.append(buf[off:off + n])
            off += (n + 7) // 8 * 8
        return out

    outs = [views(ci) for ci in counts]
    stream = torch.cuda.current_stream()

    def one_pass():
        for plan, dc, o in zip(plans, dconts, outs):
            df11.decode_batch(plan, dc, o, stream)

    # ---- timed pass (after one warm-up pass)
    one_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    log(f"stack: {n_total} weights, {resident / 1e9:.2f} GB resident compressed, "
        f"pass {ms:.2f} ms, sustained {2.0 * n_total / ms / 1e6:.1f} GB/s decoded")
    for p in plans:
        df11.check(p)

    # ---- verification pass: layer by layer into the same buffer
    host = torch.empty(buf.numel(), dtype=torch.int16, pin_memory=True)
    for gi, (plan, dc, o) in enumerate(zip(plans, dconts, outs)):
        df11.decode_batch(plan, dc, o, stream)
        df11.check(plan, stream)
        n = sum(((k + 7) // 8) * 8 for k in counts[gi])
        host[:n].copy_(buf[:n])
        h = host.numpy().view(np.uint16)
        parts, off = [], 0
        for k in counts[gi]:
            parts.append(h[off:off + k])
            off += (k + 7) // 8 * 8
        got = list(pool.map(_sha, parts))
        assert got == shas[gi], f"layer group {gi}"
    log(f"stack: all {len(groups)} layer groups bit-exact ({time.time() - t0:.1f} s)")
    pool.shutdown()
