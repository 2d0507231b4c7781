"""Stand-ins for what produces a layer's gradients chunk by chunk, so that the
update of earlier chunks can overlap the production of later ones.

"SlideDP: Scaling Host-Resident LLM Fine-Tuning Across Multiple GPUs"
(sections 核心方法 and 方法步骤详情) releases each reduced gradient chunk of a
layer to the optimizer as soon as it is ready, so that the update of finished
chunks runs while later ones are still being produced or moved. Two
producers write every chunk of every gradient replica, on the caller's
stream, with values equal to the seeded inputs (so the oracle sees the same
gradients):

- GemmProducer: matrix-core work on the GPU, a stand-in for the backward
  pass. The source chunk, viewed as an M x K matrix, times the K x K identity:
  2*M*K*K flops per chunk and replica, and the result equals the source
  exactly (each output element is one product g * 1 plus zeros, whatever the
  summation order). A tail shorter than K elements is copied.
- HostLinkProducer: DMA over the host link from pinned host memory, the
  chunked transfers of the pages' host-resident pipeline (the copy engines
  do the work; no compute unit is used).

Torch provides the GEMM, the copies and the streams; nothing here touches the
update's arithmetic.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def flat_to_layer(offsets: Sequence[int], sizes: Sequence[int], x: int) -> int:
    """Number of layer elements (tensors in order, padding excluded) that lie
    below element x of a flat per-layer gradient buffer with tensor i at
    offsets[i]."""
    return sum(min(max(x - o, 0), n) for o, n in zip(offsets, sizes))


class GemmProducer:
    """Writes dst[r] from src[r] (flat per-layer gradient buffers of equal
    length, one per replica, on the GPU) chunk by chunk.

    chunk_elems: elements of one chunk of one replica (a multiple of k);
    k: the GEMM's inner dimension (the flops per element are 2 * k)."""

    def __init__(self, src: Sequence, dst: Sequence, chunk_elems: int, k: int = 1024):
        import torch
        if chunk_elems % k:
            raise ValueError("chunk_elems must be a multiple of k")
        if len(src) != len(dst) or any(s.numel() != d.numel() for s, d in zip(src, dst)):
            raise ValueError("one source per destination, of the same length")
        self.src, self.dst, self.k, self.chunk = list(src), list(dst), k, chunk_elems
        self.eye = torch.eye(k, dtype=src[0].dtype, device=src[0].device)
        n = src[0].numel()
        self.bounds: List[Tuple[int, int]] = [(a, min(n, a + chunk_elems))
                                              for a in range(0, n, chunk_elems)]

    @property
    def flops_per_chunk(self) -> int:
        return 2 * self.chunk * self.k * len(self.src)

    def produce(self, c: int) -> None:
        """Enqueue chunk c of every replica on the current stream."""
        import torch
        a, b = self.bounds[c]
        full = (b - a) // self.k * self.k
        for s, d in zip(self.src, self.dst):
            if full:
                torch.mm(s[a:a + full].view(-1, self.k), self.eye,
                         out=d[a:a + full].view(-1, self.k))
            if a + full < b:
                d[a + full:b].copy_(s[a + full:b])


class HostLinkProducer:
    """Copies src (pinned host tensors, one per replica) into dst (flat
    per-layer gradient buffers on the GPU) chunk by chunk with asynchronous
    DMA on the caller's stream."""

    def __init__(self, src: Sequence, dst: Sequence, chunk_elems: int):
        if len(src) != len(dst) or any(s.numel() != d.numel() for s, d in zip(src, dst)):
            raise ValueError("one source per destination, of the same length")
        if not all(s.is_pinned() for s in src):
            raise ValueError("host sources must be pinned")
        self.src, self.dst, self.chunk = list(src), list(dst), chunk_elems
        n = src[0].numel()
        self.bounds: List[Tuple[int, int]] = [(a, min(n, a + chunk_elems))
                                              for a in range(0, n, chunk_elems)]

    @property
    def bytes_per_chunk(self) -> int:
        return self.chunk * self.src[0].element_size() * len(self.src)

    def produce(self, c: int) -> None:
        """Enqueue the copies of chunk c of every replica on the current stream."""
        a, b = self.bounds[c]
        for s, d in zip(self.src, self.dst):
            d[a:b].copy_(s[a:b], non_blocking=True)
