"""GPU parity of the GPU encoder (df11_encode_device): its containers must be
the oracle's byte for byte (the oracle encodes tensors up to a few hundred
thousand words in seconds; larger tensors are compared with the host
encoder, which the host tests pin to the oracle's bytes), and decode back to
the source words on the GPU."""
import numpy as np
import pytest

import oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from exponent_mixes import ENTROPY_MIXES, entropy_mix_words
from gpu_util import log

pytestmark = pytest.mark.gpu


def _gpu_encode(w, shape=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to("cuda")
    c = df11.encode_device(t.reshape(w.shape if shape is None else shape))
    return c.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 63, 64, 65, 127, 128, 129, 1000, 32767, 32768, 32769,
                               65536 + 5, 250000])
def test_edge_sizes_match_oracle_bytes(n):
    log(f"gpu encode {n}")
    w = W.normal_bf16((n,), seed=n)
    want = oracle.encode(w)
    got = _gpu_encode(w)
    assert got.size == want.size and (got == want).all()


@pytest.mark.parametrize("name", list(ENTROPY_MIXES))
def test_exponent_entropy_sweep_matches_oracle_bytes(name):
    """Code rates from 1 to 7.7 bits per element: every lane's bit count,
    the words two lanes share and the window entries, over 6 whole chunks
    and a ragged one."""
    log(f"gpu encode entropy {name}")
    w = entropy_mix_words(name, 32768 * 6 + 3001)
    want = oracle.encode(w)
    got = _gpu_encode(w)
    assert got.size == want.size and (got == want).all()


def test_special_tensors_match_oracle_bytes():
    log("gpu encode special")
    rng = np.random.default_rng(5)
    cases = [W.exhaustive_words(), rng.permutation(W.exhaustive_words()),
             np.zeros(70000, np.uint16),                                      # one symbol: 1-bit codes
             np.where(np.arange(50001) % 3 == 0, 0x3F80, 0x4000).astype(np.uint16),
             W.heavy_tail_bf16((300001,), seed=2),                             # long codes up to the cap
             np.full(1, 0x7F80, np.uint16)]
    for w in cases:
        want = oracle.encode(w)
        got = _gpu_encode(w)
        assert got.size == want.size and (got == want).all(), w.size


def test_empty_tensor_and_shapes():
    import torch
    w = np.zeros(0, np.uint16)
    assert (_gpu_encode(w) == oracle.encode(w)).all()
    w = W.normal_bf16((300, 417), seed=9)
    assert (_gpu_encode(w) == oracle.encode(w)).all()
    with pytest.raises(df11.DF11Error):   # misaligned words
        t = torch.zeros(1001, dtype=torch.int16, device="cuda")
        df11.encode_device(t[1:])


@pytest.mark.parametrize("name", ["llama8b_block", "flux_dit_block"])
def test_workloads_match_host_encoder_and_round_trip(name):
    import torch
    log(f"gpu encode workload {name}")
    for s in W.WORKLOADS[name]():
        w = s.make(threads=16)
        want = df11.encode(w.reshape(-1), shape=s.shape, threads=16)
        t = torch.from_numpy(w.view(np.int16)).to("cuda")
        c = df11.encode_device(t)
        got = c.cpu().numpy()
        assert got.size == want.size and (got == want).all(), s.name
        plan = df11.Plan([got])
        out = torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda")
        df11.decode(plan, 0, c, out)
        df11.check(plan)
        assert torch.equal(out, t.reshape(-1)), s.name


def test_batch_of_mixed_tensors_matches_single_calls():
    """One batched call (one wait on the stream) over tensors of mixed sizes,
    shapes and distributions, an empty one included: each container equals
    the oracle's."""
    import torch
    log("gpu encode batch")
    ws = [W.normal_bf16((513, 77), seed=1), np.zeros(0, np.uint16), W.heavy_tail_bf16((100003,), seed=3),
          W.exhaustive_words(), np.full(1, 0x3F80, np.uint16).reshape(()), W.normal_bf16((2 * 32768 + 9,), seed=4)]
    # (np.ascontiguousarray would give the 0-d tensor a dimension)
    ts = [torch.from_numpy(w.view(np.int16)).to("cuda") for w in ws]
    assert [t.dim() for t in ts] == [w.ndim for w in ws]
    cs = df11.encode_device_batch(ts)
    torch.cuda.synchronize()
    for w, c in zip(ws, cs):
        want = oracle.encode(w)
        got = c.cpu().numpy()
        assert got.size == want.size and (got == want).all(), w.shape


def _chunks_above_the_lds_array():
    """One exponent at probability 1/2 (a 1-bit code) and 255 uniform (9-bit
    codes), the whole tensor's words sorted by code length: the second half's
    chunks need about 9,200 stream words, more than the packing kernel's LDS
    array (8,192), so they are packed in global memory, and most of them
    start inside a word.  Returns the words and the oracle's container."""
    w = W.exponent_mix_bf16(32768 * 8 + 777, seed=24, probs=[255.0] + [1.0] * 255, e0=0)
    code_len = oracle.header(oracle.encode(w))["code_len"].astype(np.int64)
    w = w[np.argsort(code_len[(w >> 7) & 0xFF], kind="stable")]
    c = oracle.encode(w)
    h = oracle.header(c)
    ci = c[h["off_chunk_index"]:h["off_chunk_index"] + 16 * (h["n_chunks"] + 1)].view(np.uint64).reshape(-1, 2)
    b0, b1 = ci[:-1, 0].astype(np.int64), ci[1:, 0].astype(np.int64)
    nw = ((b1 - 1) >> 5) - (b0 >> 5) + 1
    assert ((nw > 8192) & (b0 % 32 != 0)).sum() >= 3
    return w, c


@pytest.mark.parametrize("fill", ["random", "ones"])
def test_containers_into_dirty_buffers_match_oracle_bytes(fill):
    """No byte of a container is cleared before the kernels run: each is
    written by exactly one kernel (stream words shared by two chunks are
    cleared by the scan kernel before the packing ORs into them).  Output
    buffers full of random bytes, or of 0xFF, must still come back as the
    oracle's bytes: long codes, chunks whose code words do not fit the
    packing kernel's LDS array (packed in global memory, with the words two
    lanes share ORed there), many chunks sharing stream words, and ragged
    tails."""
    import torch
    log(f"gpu encode into {fill} buffers")
    ws = [W.heavy_tail_bf16((5 * 32768 + 4097,), seed=21), W.exhaustive_words(),
          entropy_mix_words(sorted(ENTROPY_MIXES)[0], 9 * 32768 + 11), W.normal_bf16((33,), seed=22),
          W.normal_bf16((700001,), seed=23), _chunks_above_the_lds_array()[0]]
    ts = [torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to("cuda") for w in ws]
    if fill == "random":
        g = torch.Generator(device="cuda").manual_seed(31)
        outs = [torch.randint(0, 256, (df11.container_bound(t.numel()),), dtype=torch.uint8, device="cuda",
                              generator=g) for t in ts]
    else:
        outs = [torch.full((df11.container_bound(t.numel()),), 0xFF, dtype=torch.uint8, device="cuda")
                for t in ts]
    cs = df11.encode_device_batch(ts, outs=outs)
    torch.cuda.synchronize()
    for w, c in zip(ws, cs):
        want = oracle.encode(w)
        got = c.cpu().numpy()
        assert got.size == want.size and (got == want).all(), w.size


def test_binding_rejects_host_and_mistyped_tensors():
    """The GPU encoder reads its words on the GPU: the binding refuses host
    tensors, tensors that are not 16-bit, more than 8 dimensions and a
    wrong number of output buffers before anything reaches the library."""
    import torch
    w = torch.zeros(1000, dtype=torch.int16)
    with pytest.raises(ValueError):
        df11.encode_device(w)                                    # a host tensor
    with pytest.raises(ValueError):
        df11.encode_device(w.to(torch.int32).cuda())             # not 16-bit
    with pytest.raises(ValueError):
        df11.encode_device_batch([w.cuda(), w])                  # one on the host
    with pytest.raises(ValueError):
        df11.encode_device_batch([torch.zeros((1,) * 9, dtype=torch.int16, device="cuda")])
    with pytest.raises(ValueError):
        df11.encode_device_batch([w.cuda()], outs=[])
    with pytest.raises(ValueError):
        df11.bw_control(torch.zeros(64, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8, device="cuda"))
    # outputs of another dtype are taken as bytes
    outs = [torch.zeros((df11.container_bound(1000) + 1) // 2, dtype=torch.int16, device="cuda")]
    got = df11.encode_device_batch([w.cuda()], outs=outs)[0]
    assert (got.cpu().numpy() == oracle.encode(w.numpy().view(np.uint16))).all()
