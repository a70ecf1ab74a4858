"""A decode step over a stack of MoE layers, each preceded by a dense bf16 block.

Per layer l (batch rows b, fp32 residual stream h):

    n = bf16(RMSNorm(h))                      eps 1e-6, gain 1
    t = n; for each of the layer's dense matrices W: t = bf16(W t)
    h += t                                    } one launch
    x = bf16(RMSNorm(h))                      }
    h = moe_decode_layer_l(x, residual = h)

This is the shape of one decode step of the model described in "Kimi K3 on
GB300: 13 kernels a layer, and what 842 and 423 tokens a second measure"
(ai.thesatyajit.com), section "What one decode step of Kimi K3 does": every
layer reads a dense bf16 trunk and then its mixture-of-experts block.  The
four-matrix chain stands in for the attention block's projections.

Argument marshalling only: every step runs in libmoe_mxfp4.so's kernels.  All
buffers are allocated up front, so a step can be captured into a HIP graph.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import memory_bound_mxfp4_amd as moe


class DecodeStack:
    """Layers (packed LayerWeights) and their dense matrices (bf16 [H][H] each).

    prefetch: which upcoming weights a side stream reads into the device's
    last-level cache (moe_prefetch) while the main stream runs, the "prefetch
    on a third stream" of "Kimi K3 on GB300: 13 kernels a layer" (section
    "What the fused path changes"):
      "none"   no side stream;
      "dense"  beside MoE layer l (which leaves HBM bandwidth unused), the
               first dense matrix of layer l + 1;
      "moe"    beside the dense block of layer l, layer l's router and
               shared-expert gate/up matrices;
      "both"   both.
    The side stream only reads; the main stream never waits for it until
    the end of the step (where it joins, so a captured graph is closed)."""

    def __init__(self, layers: Sequence[moe.LayerWeights], dense: Sequence[Sequence[object]], batch: int,
                 eps: float = 1e-6, prefetch: str = "none", prefetch_blocks: int = 64):
        import torch
        if len(layers) != len(dense) or not layers:
            raise ValueError("one list of dense matrices per layer is needed")
        H = layers[0].hidden
        for w, mats in zip(layers, dense):
            if w.hidden != H or any(tuple(m.shape) != (H, H) for m in mats):
                raise ValueError("every layer and dense matrix must have the stack's hidden size")
        self.layers = list(layers)
        self.dense = [list(m) for m in dense]
        self.batch, self.hidden, self.eps = batch, H, eps
        dev = layers[0].router_w.device
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.n = torch.empty((batch, H), **bf)
        self.t = [torch.empty((batch, H), **bf), torch.empty((batch, H), **bf)]
        self.x = torch.empty((batch, H), **bf)
        k = layers[0].top_k
        self.idx = torch.empty((len(layers), batch, k), dtype=torch.int32, device=dev)
        self.gate = torch.empty((len(layers), batch, k), dtype=torch.float32, device=dev)
        self.ws = moe.alloc_workspace(layers[0], batch, dev)
        for w in layers[1:]:
            if moe.workspace_size(w, batch) > self.ws.numel():
                raise ValueError("layers of one stack must share a workspace size")
        if prefetch not in ("none", "dense", "moe", "both"):
            raise ValueError(f"unknown prefetch mode {prefetch!r}")
        self.prefetch, self.prefetch_blocks = prefetch, prefetch_blocks
        self.side = torch.cuda.Stream(device=dev) if prefetch != "none" else None

    def _side(self, main, tensors):
        """The side stream reads `tensors` once it has reached this point of `main`."""
        import torch
        ev = torch.cuda.Event()
        ev.record(main)
        self.side.wait_event(ev)
        moe.prefetch(tensors, self.prefetch_blocks, stream=self.side)

    def step(self, h, record: Optional[List[dict]] = None, stream=None):
        """One decode step over all layers; h (fp32 [batch][H]) is updated in place.
        With `record`, a dict of per-layer intermediates (device copies) is appended per layer."""
        import torch
        main = stream if stream is not None else torch.cuda.current_stream()
        n_layers = len(self.layers)
        for l, (w, mats) in enumerate(zip(self.layers, self.dense)):
            if record is not None:
                rec = {"h_in": h.clone()}
            if self.prefetch in ("moe", "both"):
                self._side(main, [w.router_w, w.shared_gate, w.shared_up])
            moe.rmsnorm_bf16(h, self.eps, out=self.n, stream=stream)
            t = self.n
            chain = []
            for j, W in enumerate(mats):
                y = self.t[j % 2]
                moe.dense_gemv_bf16(W, t, y=y, stream=stream)
                t = y
                if record is not None:
                    chain.append(y.clone())
            moe.residual_add_rmsnorm_bf16(h, t, self.eps, out=self.x, stream=stream)
            if record is not None:
                rec.update(n=self.n.clone(), chain=chain, h_mid=h.clone(), x=self.x.clone())
            if self.prefetch in ("dense", "both") and l + 1 < n_layers:
                self._side(main, [self.dense[l + 1][0]])
            moe.moe_decode_layer(w, self.x, h, idx=self.idx[l], gate=self.gate[l], ws=self.ws, stream=stream)
            if record is not None:
                rec["h_out"] = h.clone()
                record.append(rec)
        if self.side is not None:  # join: the step ends when the side stream's reads have too
            ev = torch.cuda.Event()
            ev.record(self.side)
            main.wait_event(ev)
        return h
