"""GPU parity of the just-in-time layer loop with a consumer (jit.LayerLoop):
layer l+1 decodes on its own stream while a consumer computes on layer l's
decoded weights, two BF16 buffer sets in turn (mlx-dfloat project page,
introduction: weights stay compressed in memory and each block is decoded on
the GPU as the model runs).

Checks, for three Llama-8B-shaped layers:
  * every weight the consumer sees equals the source BF16 words;
  * the consumer's products (x @ W^T for the seven tensors) equal, bit for
    bit, the same products on the original weights -- a decode that
    overwrote a buffer set still in use would change them."""
import numpy as np
import pytest

import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W

from gpu_util import log, to_device_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wgs_per_cu", [0, 2, 1])
def test_layer_loop_feeds_a_consumer_bit_exact(wgs_per_cu):
    """Also with the decode capped at two and at one workgroup per compute
    unit (the launch then has fewer workgroups than the chunks need rounds
    of, and they share the compute units with the consumer's kernels)."""
    import torch
    from lossless_bf16_weight_amd.jit import LayerLoop
    F = torch.nn.functional

    n_layers, T = 3, 64
    log(f"jit loop: {n_layers} Llama-8B-shaped layers, {T} tokens, decode workgroups per CU {wgs_per_cu}")
    groups = [W.llama8b_block(l) for l in range(n_layers)]
    words = [[s.make().reshape(-1) for s in g] for g in groups]
    conts = [[df11.encode(w, shape=s.shape) for w, s in zip(ws, g)] for ws, g in zip(words, groups)]
    loop = LayerLoop([df11.Plan(cs) for cs in conts], [[to_device_u8(c) for c in cs] for cs in conts],
                     decode_wgs_per_cu=wgs_per_cu)
    assert all(p.infos for p in loop.plans)
    assert len(loop) == n_layers

    gen = torch.Generator(device="cuda").manual_seed(0)
    x = (torch.randn(T, 4096, device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    x2 = (torch.randn(T, 14336, device="cuda", generator=gen) * 0.5).to(torch.bfloat16)

    seen, products = [], []

    def consumer(l, ws):
        seen.append([w.clone() for w in ws])
        products.append([F.linear(x2 if w.shape[1] == x2.shape[1] else x, w) for w in ws])

    loop.run(consumer)
    torch.cuda.synchronize()
    assert len(seen) == n_layers
    for l, (ws, g) in enumerate(zip(words, groups)):
        for t, (w, s) in enumerate(zip(ws, g)):
            src = torch.from_numpy(w.view(np.int16)).to("cuda").view(torch.bfloat16).view(s.shape)
            assert tuple(seen[l][t].shape) == s.shape
            assert torch.equal(seen[l][t].view(torch.int16), src.view(torch.int16)), (l, s.name)
            ref = F.linear(x2 if s.shape[1] == 14336 else x, src)
            assert torch.equal(products[l][t].view(torch.int16), ref.view(torch.int16)), (l, s.name)


def test_layer_loop_rejects_mismatched_layers():
    import torch  # noqa: F401
    from lossless_bf16_weight_amd.jit import LayerLoop
    w = W.normal_bf16((5000,), seed=1)
    c = df11.encode(w)
    p1, p2 = df11.Plan([c]), df11.Plan([c, c])
    d = to_device_u8(c)
    with pytest.raises(ValueError):
        LayerLoop([p1, p2], [[d], [d, d]])
    with pytest.raises(ValueError):
        LayerLoop([p1], [[d], [d]])


def test_plan_workgroups_per_cu_argument():
    import torch  # noqa: F401
    w = W.normal_bf16((5000,), seed=1)
    p = df11.Plan([df11.encode(w)])
    with pytest.raises(df11.DF11Error):
        p.set_wgs_per_cu(-1)
    p.set_wgs_per_cu(0)
    p.set_wgs_per_cu(64)   # above the limit: as many as fit
