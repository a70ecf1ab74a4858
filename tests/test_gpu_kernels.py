"""GPU parity of the individual entry points against the oracle:
expert_gemv_mxfp4, router_topk, and the dense-block pieces."""
import numpy as np
import pytest

import memory_bound_mxfp4_amd as moe
import oracle
import synth
from layer_inputs import bias_host, host_weights, rel_l2_rows, x_host
from synth import CONFIGS

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _mx_matrix(seed, N, K, sigma=0.02):
    w = synth.fill_f32(seed, synth.tag(9, synth.KIND_DENSE, 0, 0), sigma, N * K).reshape(N, K)
    return synth.quantise(w)


@pytest.mark.parametrize("N,K,B,xf32", [
    (64, 256, 1, False), (256, 64, 1, True), (1536, 7168, 1, False), (7168, 1536, 1, True),
    (7168, 1536, 3, True), (1536, 7168, 8, False), (100, 96, 5, False), (33, 32, 64, True), (1536, 7168, 64, False)])
def test_expert_gemv_matches_oracle(N, K, B, xf32):
    print(f"[case] gemv N={N} K={K} B={B} xf32={xf32}", flush=True)
    codes, scales = _mx_matrix(N * 7 + K, N, K)
    if xf32:
        x = synth.fill_f32(3, synth.tag(0, synth.KIND_H0), 1.0, B * K).reshape(B, K)
    else:
        x = synth.fill_bf16(3, synth.tag(0, synth.KIND_X), 1.0, B * K).reshape(B, K)
    ref = oracle.gemv_mxfp4(codes, scales, N, K, x)
    y = moe.expert_gemv_mxfp4(_dev(codes), _dev(scales), _dev(x), N, K).cpu().numpy()
    err = rel_l2_rows(y, ref)
    assert err.max() <= 1e-5, err.max()  # fp32 accumulation of exact products


def test_expert_gemv_nan_scale_poisons_its_rows():
    print("[case] gemv NaN scale", flush=True)
    N, K = 48, 128
    codes, scales = _mx_matrix(1, N, K)
    scales[5, 2] = 255
    x = synth.fill_bf16(4, synth.tag(0, synth.KIND_X), 1.0, 2 * K).reshape(2, K)
    y = moe.expert_gemv_mxfp4(_dev(codes), _dev(scales), _dev(x), N, K).cpu().numpy()
    assert np.all(np.isnan(y[:, 5]))
    assert not np.any(np.isnan(np.delete(y, 5, axis=1)))


@pytest.mark.parametrize("name,B", [("tiny", 1), ("k3_b1", 1), ("k3_b8", 8), ("k3_b64_zipf", 64), ("k3_b1", 37)])
def test_router_topk_bit_exact(name, B):
    import torch
    cfg = CONFIGS[name]
    print(f"[case] router_topk {name} B={B}", flush=True)
    hw = host_weights(cfg, 1)
    x = x_host(cfg, 1, batch=B)
    lg_ref, od = oracle.router_logits(x, hw["router_w"], hw["router_bias"], cfg.hidden, cfg.num_experts)
    idx_ref, gate_ref = oracle.topk(lg_ref, cfg.top_k)
    bias = None if hw["router_bias"] is None else _dev(hw["router_bias"])
    logits = torch.empty((B, cfg.num_experts), dtype=torch.float32, device="cuda")
    idx, gate = moe.router_topk(_dev(x), _dev(hw["router_w"]), cfg.top_k, bias=bias, logits=logits)
    assert np.array_equal(logits.cpu().numpy(), lg_ref)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.abs(gate.cpu().numpy() - gate_ref).max() <= 1e-6


def test_router_topk_ties_go_to_lower_index():
    import torch
    print("[case] router_topk ties", flush=True)
    H, E, k = 64, 40, 6
    wr = np.zeros((E, H), np.uint16)
    wr[[3, 7, 8, 30, 31, 39], 0] = 0x3F80  # six experts tie at logit 1.0 ...
    wr[[2, 20], 1] = 0x3F80               # ... two more tie at logit 1.0 via another input
    x = np.zeros((2, H), np.uint16)
    x[:, 0] = 0x3F80
    x[:, 1] = 0x3F80
    x[1, 1] = 0  # row 1: experts 2, 20 drop to 0
    idx, gate = moe.router_topk(_dev(x), _dev(wr), k)
    assert idx.cpu().numpy().tolist() == [[2, 3, 7, 8, 20, 30], [3, 7, 8, 30, 31, 39]]
    assert np.all(gate.cpu().numpy() == np.float32(1 / 6))
    # all-zero router: indices 0..k-1, gates exactly 1/k
    idx, gate = moe.router_topk(_dev(x), _dev(np.zeros((E, H), np.uint16)), 16 if E >= 16 else k)
    assert idx.cpu().numpy()[0].tolist() == list(range(16))
    assert np.all(gate.cpu().numpy() == np.float32(1 / 16))


def test_dense_pieces_match_oracle():
    import torch
    print("[case] rmsnorm / dense gemv / residual add", flush=True)
    H = 7168
    h = synth.fill_f32(2, synth.tag(0, synth.KIND_H0), 1.0, 2 * H).reshape(2, H)
    n_ref = oracle.rmsnorm_bf16(h, 1e-6)
    n = moe.rmsnorm_bf16(_dev(h), 1e-6).view(torch.int16).cpu().numpy().view(np.uint16)
    # fp32 vs double sum of squares: outputs agree to one bf16 ulp, nearly always exactly
    diff = np.abs(n.astype(np.int32) - n_ref.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 0.01
    w = synth.fill_bf16(2, synth.tag(0, synth.KIND_DENSE, 0, 0), 0.02, 512 * H).reshape(512, H)
    y_ref = oracle.dense_gemv_bf16(w, n_ref)
    y = moe.dense_gemv_bf16(_dev(w), _dev(n_ref)).view(torch.int16).cpu().numpy().view(np.uint16)
    dy = np.abs(y.astype(np.int32) - y_ref.astype(np.int32))
    assert dy.max() <= 1 and (dy > 0).mean() < 0.01
    t = np.ascontiguousarray(np.tile(y_ref, (1, H // 512)))
    hh = _dev(h.copy())
    moe.residual_add_bf16(hh, _dev(t))
    ref = h + (t.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(hh.cpu().numpy(), ref)
    # the fused add + norm equals the two launches bit for bit
    h2 = _dev(h.copy())
    x2 = moe.residual_add_rmsnorm_bf16(h2, _dev(t), 1e-6)
    assert np.array_equal(h2.cpu().numpy(), ref)
    x1 = moe.rmsnorm_bf16(hh, 1e-6)
    assert torch.equal(x1, x2)


@pytest.mark.parametrize("B", [1, 2, 8, 17, 64])
@pytest.mark.parametrize("N,K", [(512, 7168), (100, 520)])
def test_dense_gemv_batches_match_oracle(B, N, K):
    """dense_gemv_bf16 at every batch shape (one row on the vector ALU, 2..64
    rows on the matrix cores; ragged N and K): each output within one bf16
    ulp of the oracle's rounding of the exact sum, and nearly always equal."""
    import torch
    print(f"[case] dense gemv B{B} N{N} K{K}", flush=True)
    w = synth.fill_bf16(3, synth.tag(0, synth.KIND_DENSE, 0, 1), 0.02, N * K).reshape(N, K)
    x = synth.fill_bf16(3, synth.tag(0, synth.KIND_X, 0, B), 1.0, B * K).reshape(B, K)
    y_ref = oracle.dense_gemv_bf16(w, x)
    y = moe.dense_gemv_bf16(_dev(w), _dev(x)).view(torch.int16).cpu().numpy().view(np.uint16)
    dy = np.abs(y.astype(np.int32) - y_ref.astype(np.int32))
    assert dy.max() <= 1 and (dy > 0).mean() < 0.01, (int(dy.max()), float((dy > 0).mean()))
