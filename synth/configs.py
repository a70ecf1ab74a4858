"""The five synthetic workloads of the MoE decode layer (inputs only).

Each workload fixes the layer shape, the batch, the value distributions and
the seed recipe; nothing here computes any part of the layer.

* ``tiny``        hidden 256, 16 experts, expert intermediate 64, top-2, one
                  bf16 shared expert of intermediate 64, batch 1; router and
                  activations ~N(0,1), expert and shared weights ~N(0,0.02).
* ``k3_b1``       Kimi-K3-shaped layer: hidden 7168, 896 experts, top-16,
                  intermediate 1536 (17,547,264-byte MXFP4 experts), one bf16
                  shared expert of intermediate 1536, batch 1; all weights
                  ~N(0,0.02), activations ~N(0,1).
* ``k3_b8``       the same layer at batch 8 (one anchor + 7 draft rows of a
                  speculative verify step), rows drawn independently.
* ``k3_b64_zipf`` the same layer at batch 64 with a Zipf-like router bias
                  b_e = -1.1 ln(rank_e) (rank: seeded permutation of 1..896).
* ``k3_stack8``   8 consecutive K3-shaped layers at batch 1, each preceded by
                  a chain of 4 bf16 7168x7168 dense GEMVs with RMSNorm
                  (eps 1e-6); the residual stream enters as fp32 N(0,1).

The layer sizes and per-expert byte count follow "Kimi K3 on GB300: 13
kernels a layer, and what 842 and 423 tokens a second measure"
(ai.thesatyajit.com), section "What one decode step of Kimi K3 does"; the
batch-8 verify shape follows its section "What DSpark adds".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    shared_inter: int
    batch: int
    router_sigma: float
    weight_sigma: float = 0.02
    x_sigma: float = 1.0
    zipf_s: Optional[float] = None
    layers: int = 1
    dense_mats: int = 0
    rms_eps: float = 1e-6


CONFIGS = {
    "tiny": LayerConfig("tiny", 256, 64, 16, 2, 64, 1, router_sigma=1.0),
    "k3_b1": LayerConfig("k3_b1", 7168, 1536, 896, 16, 1536, 1, router_sigma=0.02),
    "k3_b8": LayerConfig("k3_b8", 7168, 1536, 896, 16, 1536, 8, router_sigma=0.02),
    "k3_b64_zipf": LayerConfig("k3_b64_zipf", 7168, 1536, 896, 16, 1536, 64, router_sigma=0.02, zipf_s=1.1),
    "k3_stack8": LayerConfig("k3_stack8", 7168, 1536, 896, 16, 1536, 1, router_sigma=0.02, layers=8, dense_mats=4),
}
