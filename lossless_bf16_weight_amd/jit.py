"""Just-in-time decode of a resident compressed layer stack, one layer ahead
of its consumer.

The compressed containers of every layer stay in device memory.  BF16 weights
exist only for two layers at a time: the one the consumer is using and the
next one, which is decoded meanwhile on a stream of its own (mlx-dfloat
project page, introduction: the weights stay compressed in memory and each
block is decoded on the GPU as the model runs).  Orchestration only: every
decode runs in libdf11's kernel, every consumer computation is the caller's.
"""
from __future__ import annotations

from typing import Callable, List, Sequence

import torch

from ._lib import Plan, decode_batch


class LayerLoop:
    """Decode layer l+1 while `consumer(l, weights)` runs layer l.

    decode_wgs_per_cu caps the decode's workgroups per compute unit for every
    layer's plan (0: as many as fit): with 2, the decode shares the compute
    units with a small consumer (one token's matrix-vector products) instead
    of running after it; with large consumers the default is faster.

    plans[l] is the plan of layer l and containers[l] its device containers
    (uint8 tensors, one per planned tensor).  Every layer has the same number
    of tensors; buffer t of each of the two buffer sets is sized for the
    largest tensor t over the layers, and a layer's weights are views of it
    with the tensor's shape (dtype bfloat16)."""

    def __init__(self, plans: Sequence[Plan], containers: Sequence[Sequence[torch.Tensor]],
                 device: str = "cuda", decode_wgs_per_cu: int = 0):
        if len(plans) == 0 or len(plans) != len(containers):
            raise ValueError("one plan and one container list per layer")
        n_t = plans[0].n_tensors
        for p, cs in zip(plans, containers):
            if p.n_tensors != n_t or len(cs) != n_t:
                raise ValueError("every layer needs the same number of tensors")
        self.plans = list(plans)
        # decode workgroups per compute unit (0: as many as fit).  Fewer leave
        # room on every compute unit for the consumer's kernels, so that the
        # next layer's decode runs beside them instead of after them.
        self.set_decode_wgs_per_cu(decode_wgs_per_cu)
        self.containers = [list(cs) for cs in containers]
        self.shapes = [[tuple(int(d) for d in p.infos[t]["dims"]) or (1,) for t in range(n_t)]
                       for p in self.plans]
        self.sizes = [[int(p.infos[t]["n_elems"]) for t in range(n_t)] for p in self.plans]
        biggest = [max(self.sizes[l][t] for l in range(len(plans))) for t in range(n_t)]
        self.buffers = [[torch.empty(max(b, 1), dtype=torch.bfloat16, device=device) for b in biggest]
                        for _ in range(2)]
        self.decode_stream = torch.cuda.Stream(device=device)

    def set_decode_wgs_per_cu(self, n: int) -> None:
        """Cap the decode's workgroups per compute unit (0: as many as fit)."""
        self.decode_wgs_per_cu = int(n)
        for p in self.plans:
            p.set_wgs_per_cu(self.decode_wgs_per_cu)

    def __len__(self) -> int:
        return len(self.plans)

    def weights(self, slot: int, layer: int) -> List[torch.Tensor]:
        """Views of buffer set `slot` as layer `layer`'s tensors."""
        return [self.buffers[slot][t][:n].view(shape)
                for t, (n, shape) in enumerate(zip(self.sizes[layer], self.shapes[layer]))]

    def decode_into(self, layer: int, slot: int, stream) -> None:
        """Enqueue layer `layer`'s decode into buffer set `slot` on `stream`."""
        outs = [self.buffers[slot][t][:n] for t, n in enumerate(self.sizes[layer])]
        decode_batch(self.plans[layer], self.containers[layer], outs, stream=stream)

    def run(self, consumer: Callable[[int, List[torch.Tensor]], None], compute_stream=None) -> None:
        """Run consumer(l, weights of layer l) on the compute stream for every
        layer in order, each layer's decode enqueued one layer ahead on the
        decode stream.  Returns once everything is enqueued."""
        cs = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        ds = self.decode_stream
        decoded = [torch.cuda.Event(), torch.cuda.Event()]
        consumed = [torch.cuda.Event(), torch.cuda.Event()]
        ds.wait_stream(cs)   # whatever the caller enqueued before (inputs, buffers) comes first
        self.decode_into(0, 0, ds)
        decoded[0].record(ds)
        for l in range(len(self.plans)):
            s = l & 1
            if l + 1 < len(self.plans):
                ns = s ^ 1
                if l >= 1:
                    ds.wait_event(consumed[ns])   # layer l-1's consumer is done with that set
                self.decode_into(l + 1, ns, ds)
                decoded[ns].record(ds)
            cs.wait_event(decoded[s])
            with torch.cuda.stream(cs):
                consumer(l, self.weights(s, l))
            consumed[s].record(cs)
        cs.wait_stream(ds)
