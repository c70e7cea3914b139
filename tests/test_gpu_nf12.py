"""GPU parity of the NF12 decode kernel (df11_nf12_decode) against the NF12
oracle and the source words: edge sizes with guard words around every
output, every 16-bit word, outlier-heavy tensors, the five workloads (the
stack's embedding and a sample of its layers), a corrupted container (the
kernel stays inside its buffers) and bad arguments."""
import numpy as np
import pytest

from oracle import nf12 as nf12_oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from exponent_mixes import ENTROPY_MIXES, entropy_mix_words, random_exponent_case
from gpu_util import empty_words, log, to_device_u8

pytestmark = pytest.mark.gpu


def _decode(c, n, guard=32):
    import torch
    buf, out = empty_words(n, guard=guard)
    df11.nf12_decode(c[:256], to_device_u8(c), out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy().view(np.uint16)
    assert (host[:guard] == 0x5A5A).all() and (host[guard + n:] == 0x5A5A).all(), "wrote outside the output"
    return host[guard:guard + n]


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 15, 63, 64, 65, 511, 512, 513, 2047, 2048, 2049,
                               8191, 8193, 65536 + 5, 1000003])
def test_edge_sizes_bit_exact(n):
    log(f"nf12 size {n}")
    w = W.normal_bf16((n,), seed=n)
    w[::53] = 0                       # outlier groups spread through the tensor
    c = df11.nf12_encode(w)
    got = _decode(c, n)
    assert (got == w).all()
    assert (got == nf12_oracle.decode(c, n)).all()


@pytest.mark.parametrize("name", list(ENTROPY_MIXES))
def test_exponent_spread_sweep(name):
    """Exponent distributions from 2 to 200 values: from no escaped group to
    nearly all groups escaped, against the oracle and the source words."""
    log(f"nf12 exponent spread {name}")
    n = 100000 + 13
    w = entropy_mix_words(name, n)
    c = df11.nf12_encode(w)
    got = _decode(c, n)
    assert (got == w).all()
    assert (got == nf12_oracle.decode(c, n)).all()


def test_every_word_and_all_outliers():
    log("nf12 every word")
    for w in (W.exhaustive_words(), np.random.default_rng(0).permutation(W.exhaustive_words()),
              np.zeros(4096 + 3, np.uint16), np.full(4099, 0x3F80, np.uint16)):
        c = df11.nf12_encode(w)
        assert (_decode(c, w.size) == w).all()


def test_empty_tensor_enqueues_nothing():
    import torch
    c = df11.nf12_encode(np.zeros(0, np.uint16))
    out = torch.full((8,), 0x5A5A, dtype=torch.int16, device="cuda")
    df11.nf12_decode(c[:256], to_device_u8(np.pad(c, (0, 16))), out)
    torch.cuda.synchronize()
    assert (out.cpu().numpy().view(np.uint16) == 0x5A5A).all()


@pytest.mark.parametrize("name", ["single_2048", "llama8b_block", "heavy_tail_8192", "flux_dit_block"])
def test_workloads_bit_exact(name):
    import torch
    log(f"nf12 workload {name}")
    for s in W.WORKLOADS[name]():
        w = s.make().reshape(-1)
        c = df11.nf12_encode(w, threads=16)
        out = torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda")
        df11.nf12_decode(c[:256], to_device_u8(c), out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        assert (got == w).all(), s.name
        # the oracle on a sample of groups: decode a slice of the container's
        # groups by re-encoding the matching slice of words
        lo = (w.size // 3) // 512 * 512
        part = w[lo:lo + 4096]
        assert (nf12_oracle.decode(nf12_oracle.encode(part), part.size) == got[lo:lo + part.size]).all()


def test_llama8b_stack_sample_bit_exact():
    """The stack's embedding and three of its 32 layers."""
    import torch
    log("nf12 stack sample")
    groups = W.llama8b_stack_layers(32)
    for g in (groups[0], groups[17], groups[31], groups[32]):
        for s in g:
            w = s.make().reshape(-1)
            c = df11.nf12_encode(w, threads=16)
            out = torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda")
            df11.nf12_decode(c[:256], to_device_u8(c), out)
            torch.cuda.synchronize()
            assert (out.cpu().numpy().view(np.uint16) == w).all(), s.name


def test_corrupted_flags_stay_in_bounds():
    """Every flag bit set on the device copy (the header unchanged): lanes
    read escape entries clamped into the escape buffer; the words differ,
    nothing outside the output is written."""
    import torch
    log("nf12 corrupted flags")
    w = W.normal_bf16((8 * 5000 + 3,), seed=11)
    w[::997] = 0
    c = df11.nf12_encode(w)
    h = nf12_oracle.header(c)
    bad = c.copy()
    n_words = (h["n_groups"] + 63) // 64
    bad[h["off_flags"]:h["off_flags"] + 8 * n_words] = 0xFF
    buf, out = empty_words(w.size, guard=32)
    df11.nf12_decode(c[:256], to_device_u8(bad), out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy().view(np.uint16)
    assert (host[:32] == 0x5A5A).all() and (host[32 + w.size:] == 0x5A5A).all()
    assert not (host[32:32 + w.size] == w).all()


def test_bad_arguments_are_rejected():
    import torch
    w = W.normal_bf16((4096,), seed=1)
    c = df11.nf12_encode(w)
    dc = to_device_u8(c)
    out = torch.full((w.size + 8,), 0x5A5A, dtype=torch.int16, device="cuda")
    with pytest.raises(df11.DF11Error):
        hdr = c[:256].copy()
        hdr[0] = ord("X")
        df11.nf12_decode(hdr, dc, out)
    with pytest.raises(df11.DF11Error):
        df11.nf12_decode(c[:256], dc, out[1:])          # misaligned output
    with pytest.raises(ValueError):
        df11.nf12_decode(c[:100], dc, out)
    # what the binding checks before the call (the library cannot see the
    # size of a device buffer)
    with pytest.raises(ValueError):
        df11.nf12_decode(c[:256], dc, out[:w.size - 8])  # output too small
    with pytest.raises(ValueError):
        df11.nf12_decode(c[:256], dc[:-16], out)        # container too short
    with pytest.raises(ValueError):
        df11.nf12_decode_batch([c[:256]], [dc], [out.view(torch.int32)])   # not 16-bit words


def test_batch_of_mixed_sizes_split_over_launches():
    """30 tensors (more than one launch holds), mixed sizes including empty
    and partial groups, guard words around every output."""
    import torch
    log("nf12 batch of 30")
    sizes = [0, 1, 9, 4096, 65536 + 7, 513, 8, 100003] + [3000 + 131 * i for i in range(22)]
    ws = []
    for i, n in enumerate(sizes):
        w = W.normal_bf16((n,), seed=100 + i)
        if n:
            w[::(17 + i)] = 0
        ws.append(w)
    cs = [df11.nf12_encode(w) for w in ws]
    bufs = [empty_words(max(n, 1), guard=32) for n in sizes]
    dcs = [to_device_u8(np.pad(c, (0, 16))) for c in cs]
    df11.nf12_decode_batch([c[:256] for c in cs], dcs, [o for _, o in bufs])
    torch.cuda.synchronize()
    for w, (buf, _), n in zip(ws, bufs, sizes):
        host = buf.cpu().numpy().view(np.uint16)
        assert (host[32:32 + n] == w).all()
        assert (host[:32] == 0x5A5A).all() and (host[32 + max(n, 1):] == 0x5A5A).all()


def test_random_distributions_batched():
    """60 seeded random exponent distributions (random sizes, from no
    escaped group to all of them) in the NF12 oracle's containers, decoded
    in one batched call with guard words around every output."""
    import torch
    log("nf12 random distributions")
    ws = [random_exponent_case(seed, 120_000) for seed in range(60)]
    cs = [nf12_oracle.encode(w) for w in ws]
    bufs = [empty_words(max(w.size, 1), guard=32) for w in ws]
    dcs = [to_device_u8(np.pad(c, (0, 16))) for c in cs]
    df11.nf12_decode_batch([c[:256] for c in cs], dcs, [o for _, o in bufs])
    torch.cuda.synchronize()
    for seed, (w, (buf, _)) in enumerate(zip(ws, bufs)):
        host = buf.cpu().numpy().view(np.uint16)
        assert (host[32:32 + w.size] == w).all(), seed
        assert (host[:32] == 0x5A5A).all() and (host[32 + max(w.size, 1):] == 0x5A5A).all(), seed
