"""HIP-graph capture of a fixed-shape k-MIP forward + backward.

Small graphs are launch-bound: one forward and backward is some two dozen
short kernels.  Recording them once into a HIP graph (through
torch.cuda.CUDAGraph, which captures the library's launches on the capture
stream) and replaying it removes the per-launch host cost.  libkmip records
no memset nodes (it clears memory with its own kernels) and allocates
nothing, so every buffer here is allocated before capture and reused by
every replay.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import kmip


class CapturedKmip:
    """Static buffers plus one captured forward (and optionally backward).

    Copy new inputs into `q`, `k`, `v` (and `dout`) in place, call replay(),
    read `out`, `topk_idx`, `topk_score` (and `dq`, `dk`, `dv`).
    """

    def __init__(self, N: int, H: int, d: int, topk: int,
                 graph_offsets: Optional[torch.Tensor] = None, backward: bool = True,
                 device: str = "cuda"):
        dev = torch.device(device)
        self.topk = topk
        self.graph_offsets = graph_offsets
        B = 0 if graph_offsets is None else int(graph_offsets.numel()) - 1
        bf = dict(dtype=torch.bfloat16, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.q = torch.zeros((N, H, d), **bf)
        self.k = torch.zeros((N, H, d), **bf)
        self.v = torch.zeros((N, H, d), **bf)
        self.out = torch.empty((N, H, d), **f32)
        self.topk_idx = torch.empty((N, H, topk), dtype=torch.int32, device=dev)
        self.topk_score = torch.empty((N, H, topk), **f32)
        self.fws = torch.empty(max(1, kmip.forward_workspace_bytes(N, H, d, topk, B)),
                               dtype=torch.uint8, device=dev)
        self.backward = backward
        if backward:
            self.dout = torch.zeros((N, H, d), **f32)
            self.dq = torch.empty((N, H, d), **f32)
            self.dk = torch.empty((N, H, d), **f32)
            self.dv = torch.empty((N, H, d), **f32)
            self.bws = torch.empty(max(1, kmip.backward_workspace_bytes(N, H, d, topk, B)),
                                   dtype=torch.uint8, device=dev)
        # One eager run on a side stream first (as torch recommends before
        # capture), then the capture itself.
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            self._step(s)
        torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step(torch.cuda.current_stream(dev))

    def _step(self, stream):
        kmip.forward(self.q, self.k, self.v, self.topk, self.graph_offsets, out=self.out,
                     topk_idx=self.topk_idx, topk_score=self.topk_score, workspace=self.fws,
                     stream=stream)
        if self.backward:
            kmip.backward(self.q, self.k, self.v, self.topk, self.topk_idx, self.topk_score,
                          self.dout, self.graph_offsets, dq=self.dq, dk=self.dk, dv=self.dv,
                          workspace=self.bws, stream=stream)

    def replay(self):
        self.graph.replay()
