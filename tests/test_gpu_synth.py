"""The generator's device build writes the same bytes as its host build."""
import numpy as np
import pytest

import synth
import memory_bound_mxfp4_amd as moe
from layer_inputs import device_weights, host_weights, host_experts
from test_pack import pack_ref
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def test_tiny_layer_bytes_match_host():
    import torch
    cfg = CONFIGS["tiny"]
    print("[case] synth twin tiny seed 5", flush=True)
    w = device_weights(cfg, 5, packed=False)
    hw = host_weights(cfg, 5)
    assert np.array_equal(w.router_w.cpu().numpy().view(np.uint16), hw["router_w"])
    assert np.array_equal(w.shared_down.cpu().numpy().view(np.uint16), hw["shared_down"])
    blobs = w.experts.cpu().numpy().reshape(cfg.num_experts, -1)
    ex = host_experts(cfg, 5, range(cfg.num_experts))
    for e in range(cfg.num_experts):
        assert np.array_equal(blobs[e], ex[e]), e


def test_k3_sampled_bytes_match_host(k3_layer):
    cfg = CONFIGS["k3_b1"]
    print("[case] synth twin K3 seed 0 sampled experts", flush=True)
    nb = synth.expert_bytes(cfg.hidden, cfg.inter)
    # the shared fixture holds the experts packed for the layer kernel
    assert k3_layer.expert_layout == moe.MOE_EXPERTS_PACKED
    for e in (0, 447, 895):
        dev = k3_layer.experts[e * nb:(e + 1) * nb].cpu().numpy()
        assert np.array_equal(dev, pack_ref(synth.expert_blob(0, 0, e, cfg.hidden, cfg.inter, 0.02), cfg.hidden,
                                            cfg.inter)), e
    rw = k3_layer.router_w[100:104].cpu().numpy().view(np.uint16)
    assert np.array_equal(rw, synth.bf16_rows(0, synth.tag(0, synth.KIND_ROUTER), 0.02, cfg.hidden, 100, 4))
    sg = k3_layer.shared_gate[1535].cpu().numpy().view(np.uint16)
    assert np.array_equal(sg, synth.bf16_rows(0, synth.tag(0, synth.KIND_SHARED, 0, 0), 0.02, cfg.hidden, 1535, 1)[0])
