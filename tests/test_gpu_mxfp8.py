"""GPU parity of moe_decode_layer_mxfp8 (routed experts as FP4 x MXFP8, the
precision of the expert kernel in "Kimi K3 on GB300", section "Why batch 1
on a rack is not only a bandwidth problem") against the oracle's MXFP8
variant: expert indices and gates bit-identical to the oracle's (and to
moe_decode_layer's), outputs within TOL_MX8 relative L2 per row on every row.

TOL_MX8 follows from the arithmetic.  The activations entering FC1 are bf16,
so both sides quantise them to the same MXFP8 codes; FC1 then differs only
in summation order (fp32 on the matrix cores, double in the oracle), about
1e-6 relative.  The SwiGLU output entering FC2 is quantised from those two
slightly different fp32 values, so an element lying within that difference
of an E4M3 rounding boundary lands on neighbouring codes on the two sides:
one E4M3 step, at most 2^-3 of the element, i.e. about 2^-3 / sqrt(I) ~ 3e-3
of that slot's output for a typical element, diluted by the gate (~1/16)
and the other slots in the row's MoE sum.  A few such flips per row stay
well inside 1e-2; TOL_MX8 = 1e-2 on the output and on the MoE delta.
"""
import numpy as np
import pytest

import memory_bound_mxfp4_amd as moe
import oracle
import synth
from layer_inputs import device_weights, host_experts, host_weights, rel_l2_rows, residual_from_x, x_host
from synth import CONFIGS

pytestmark = pytest.mark.gpu
TOL_MX8 = 1e-2


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _oracle_mx8(cfg, seed, x, res, bias=None):
    hw = host_weights(cfg, seed)
    lg, _ = oracle.router_logits(x, hw["router_w"], bias, cfg.hidden, cfg.num_experts)
    idx, _ = oracle.topk(lg, cfg.top_k)
    experts = host_experts(cfg, seed, idx.ravel())
    return oracle.moe_layer(cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.shared_inter, hw["router_w"],
                            bias, hw["shared_gate"], hw["shared_up"], hw["shared_down"], experts, x, res, mx8=True)


def _run_both(w, x, res):
    import torch
    r8 = _dev(res.copy())
    idx8, gate8 = moe.moe_decode_layer(w, _dev(x), r8, mxfp8=True)
    r = _dev(res.copy())
    idx, gate = moe.moe_decode_layer(w, _dev(x), r)
    torch.cuda.synchronize()
    assert torch.equal(idx8, idx) and torch.equal(gate8.view(torch.int32), gate.view(torch.int32))
    return r8.cpu().numpy(), idx8.cpu().numpy(), gate8.cpu().numpy(), r.cpu().numpy()


def _check(ref, x, res, out, idx, gate, exact_out):
    assert np.array_equal(idx, ref["idx"])
    assert np.abs(gate - ref["gate"]).max() <= 1e-6
    err = rel_l2_rows(out, ref["out"])
    delta = rel_l2_rows(out - res, ref["out"] - res)
    vs_exact = rel_l2_rows(out - res, exact_out - res)
    print(f"    max rel-L2 vs MXFP8 oracle: out {err.max():.3e} moe-delta {delta.max():.3e} "
          f"(median {np.median(delta):.3e}); MoE delta vs the exact path {vs_exact.max():.3e}", flush=True)
    assert err.max() <= TOL_MX8
    assert delta.max() <= TOL_MX8


@pytest.mark.parametrize("B", [1, 3, 5, 64])
def test_mx8_tiny_layer(B):
    cfg = CONFIGS["tiny"]
    print(f"[case] mxfp8 layer tiny B{B}", flush=True)
    w = device_weights(cfg, 3)
    x = x_host(cfg, 3, batch=B)
    res = residual_from_x(x)
    out, idx, gate, exact = _run_both(w, x, res)
    _check(_oracle_mx8(cfg, 3, x, res), x, res, out, idx, gate, exact)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", [1, 8, 33])
def test_mx8_k3(k3_layer, B):
    cfg = CONFIGS["k3_b8"]
    print(f"[case] mxfp8 layer K3 B{B}", flush=True)
    x = x_host(cfg, 0, variant=9, batch=B)
    res = residual_from_x(x)
    out, idx, gate, exact = _run_both(k3_layer, x, res)
    _check(_oracle_mx8(cfg, 0, x, res), x, res, out, idx, gate, exact)


@pytest.mark.timeout(900)
def test_mx8_k3_batch64_zipf(k3_layer):
    cfg = CONFIGS["k3_b64_zipf"]
    print("[case] mxfp8 layer K3 B64 zipf", flush=True)
    bias = synth.zipf_bias(0, 0, cfg.num_experts, cfg.zipf_s)
    k3_layer.router_bias = _dev(bias)
    try:
        x = x_host(cfg, 0)
        res = residual_from_x(x)
        out, idx, gate, exact = _run_both(k3_layer, x, res)
    finally:
        k3_layer.router_bias = None
    _check(_oracle_mx8(cfg, 0, x, res, bias=bias), x, res, out, idx, gate, exact)


def test_mx8_deterministic_and_status(k3_layer):
    import torch
    cfg = CONFIGS["k3_b8"]
    print("[case] mxfp8 layer K3 B8 determinism x10", flush=True)
    x = _dev(x_host(cfg, 0, variant=11))
    res0 = _dev(residual_from_x(x_host(cfg, 0, variant=11)))
    ws = moe.alloc_workspace(k3_layer, 8)
    first = None
    for _ in range(10):
        r = res0.clone()
        moe.moe_decode_layer(k3_layer, x, r, ws=ws, mxfp8=True)
        torch.cuda.synchronize()
        first = r.view(torch.int32).clone() if first is None else first
        assert torch.equal(r.view(torch.int32), first)
    assert moe.workspace_status(ws) == 0
