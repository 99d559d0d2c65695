"""A stack of routed-expert layers run back to back on one stream, eagerly
or as one captured HIP graph (the decode-graph pattern of the MXFP4-FP8-R12
card's runtime, "decode CUDA graphs" in its deployment table).

Plumbing only: every kernel is a moe_fp4_forward launch of the library; torch
supplies the device buffers, the stream and the graph object.  All buffers
(inputs, routing, outputs, one shared workspace) are allocated before capture,
so a replay allocates nothing and launches exactly the kernels of an eager
pass (the forward issues no memset or host synchronisation)."""
from __future__ import annotations

from typing import List, Optional

import torch

from ._lib import MoELayer, moe_forward, workspace_size


class LayerStack:
    def __init__(self, layers: List[MoELayer], xs: List[torch.Tensor], ids: List[torch.Tensor],
                 weights: List[torch.Tensor]):
        assert len(layers) == len(xs) == len(ids) == len(weights) and layers
        self.layers, self.xs, self.ids, self.weights = layers, xs, ids, weights
        dev = xs[0].device
        need = max(workspace_size(l, int(x.shape[0])) for l, x in zip(layers, xs))
        self.workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        self.ys = [torch.empty(int(x.shape[0]), l.hidden, dtype=torch.float32, device=dev)
                   for l, x in zip(layers, xs)]
        self.graph: Optional[torch.cuda.CUDAGraph] = None

    def eager(self):
        """One pass over the layers on the current stream."""
        for l, x, i, w, y in zip(self.layers, self.xs, self.ids, self.weights, self.ys):
            moe_forward(l, x, i, w, self.workspace, y)

    def capture(self):
        """Capture one pass as a graph (after an eager pass has set every
        kernel's launch attributes)."""
        self.eager()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.eager()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = g

    def replay(self):
        assert self.graph is not None, "capture() first"
        self.graph.replay()
