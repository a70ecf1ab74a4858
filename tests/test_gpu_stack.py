"""GPU parity of the 8-layer decode-step stack (dense bf16 block + MoE layer
per layer), teacher-forced: each step of layer l is checked against the
oracle on the inputs the GPU itself produced for it, because bf16 rounding
of the norms and GEMV outputs turns last-bit differences into one-ulp input
changes that a free-running comparison would carry into later layers (and
into near-tie routing decisions).  Layer 0's inputs come straight from the
generator, so its check is free of teacher forcing.

Dense GEMV and RMSNorm outputs are bf16 roundings of fp32 (GPU) vs double
(oracle) sums: equal to one bf16 ulp, and exactly equal almost always.
Expert indices must match exactly; layer outputs within 2e-3 relative L2."""
import numpy as np
import pytest

import oracle
from layer_inputs import dense_host, h0_host, host_weights, oracle_layer, rel_l2_rows
from synth import CONFIGS

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_close(got, ref, what):
    """got and ref are bf16 roundings of the same fp32 (GPU) / double (oracle)
    sum: within one bf16 ulp of ref, or -- where the sum cancels to a value
    far below the row's scale, so an ulp of it is tiny -- within 2^-16 of the
    row's RMS (fp32 accumulation error over ~7k terms is ~1e-6 of that
    scale); and bit-equal almost everywhere."""
    g, r = _f32(got), _f32(ref)
    ulp = np.where(r != 0, np.exp2(np.floor(np.log2(np.abs(r) + 1e-300)) - 7), 0.0)
    floor = 2.0 ** -16 * np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    bad = np.abs(g - r) > np.maximum(ulp, floor)
    assert not bad.any(), (what, float(np.abs(g - r)[bad].max()), float(floor.max()))
    assert (got != ref).mean() < 0.01, (what, float((got != ref).mean()))


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(900)
def test_stack_teacher_forced(k3_stack):
    import torch
    cfg = CONFIGS["k3_stack8"]
    print("[case] stack 8 layers, teacher-forced", flush=True)
    h = torch.from_numpy(h0_host(cfg, 0)).cuda()
    record = []
    k3_stack.step(h, record=record)
    torch.cuda.synchronize()
    idx_all = k3_stack.idx.cpu().numpy()
    assert np.array_equal(record[0]["h_in"].cpu().numpy(), h0_host(cfg, 0))
    for l, rec in enumerate(record):
        h_in = rec["h_in"].cpu().numpy()
        n = _bits(rec["n"])
        _bf16_close(n, oracle.rmsnorm_bf16(h_in, cfg.rms_eps), f"rmsnorm l{l}")
        t_prev = n
        for j, y_dev in enumerate(rec["chain"]):
            y = _bits(y_dev)
            _bf16_close(y, oracle.dense_gemv_bf16(dense_host(cfg, 0, l, j), t_prev), f"dense l{l} j{j}")
            t_prev = y
        h_mid = rec["h_mid"].cpu().numpy()
        assert np.array_equal(h_mid, h_in + (t_prev.astype(np.uint32) << 16).view(np.float32)), l
        x = _bits(rec["x"])
        _bf16_close(x, oracle.rmsnorm_bf16(h_mid, cfg.rms_eps), f"rmsnorm2 l{l}")
        hw = host_weights(cfg, 0, l)
        lg, _ = oracle.router_logits(x, hw["router_w"], hw["router_bias"], cfg.hidden, cfg.num_experts)
        idx_ref, _ = oracle.topk(lg, cfg.top_k)
        assert np.array_equal(idx_all[l], idx_ref), l
        ref = oracle_layer(cfg, 0, x, h_mid, layer=l)
        err = rel_l2_rows(rec["h_out"].cpu().numpy(), ref["out"]).max()
        print(f"    layer {l}: rel-L2 {err:.3e}", flush=True)
        assert err <= TOL
    print(f"    layers checked: {len(record)}", flush=True)


def test_stack_graph_replay_matches_eager(k3_stack):
    """The whole step captured in a HIP graph: every replay equals the eager step."""
    import torch
    cfg = CONFIGS["k3_stack8"]
    print("[case] stack graph replay x3 vs eager", flush=True)
    h0 = torch.from_numpy(h0_host(cfg, 0)).cuda()
    h = h0.clone()
    k3_stack.step(h)
    torch.cuda.synchronize()
    eager = h.cpu().numpy()
    eager_idx = k3_stack.idx.cpu().numpy()
    hg = h0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        k3_stack.step(hg, stream=s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        k3_stack.step(hg, stream=s)
    for rep in range(3):
        hg.copy_(h0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(hg.cpu().numpy().view(np.uint32), eager.view(np.uint32)), rep
        assert np.array_equal(k3_stack.idx.cpu().numpy(), eager_idx), rep


def test_stack_with_side_stream_prefetch_matches(k3_stack):
    """The side-stream prefetch only reads: a step with it (eager and as a
    replayed HIP graph) equals the plain step bit for bit."""
    import torch
    from memory_bound_mxfp4_amd.stack import DecodeStack
    cfg = CONFIGS["k3_stack8"]
    print("[case] stack with side-stream prefetch vs plain", flush=True)
    h0 = torch.from_numpy(h0_host(cfg, 0)).cuda()
    ref = h0.clone()
    k3_stack.step(ref)
    torch.cuda.synchronize()
    pf = DecodeStack(k3_stack.layers, k3_stack.dense, cfg.batch, cfg.rms_eps, prefetch="both")
    h = h0.clone()
    pf.step(h)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int32), ref.view(torch.int32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    hg = h0.clone()
    with torch.cuda.stream(s):
        pf.step(hg, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pf.step(hg, stream=s)
    for rep in range(3):
        hg.copy_(h0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(hg.view(torch.int32), ref.view(torch.int32)), rep
