"""Pins of the oracle's SwiGLU experts, the combine into the residual, and the
dense-block pieces (bf16 rounding, RMSNorm, bf16 GEMV).

Closed forms used: with a one-hot activation the gate and up GEMVs reduce to
reading one decoded column, so an expert's output reduces to
W_down (silu(g) * u) with silu(z) = z * logistic(z) taken from scipy's expit;
silu(z) - silu(-z) = z for every z; with every routed expert equal the gate
weights (which sum to 1) drop out; with k = E the renormalised top-k gates are
the plain softmax (scipy).  The layer's structure -- router, shared expert,
16 routed experts summed into the residual -- is the per-layer work list of
"Kimi K3 on GB300: 13 kernels a layer" (section "What one decode step of Kimi
K3 does").
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle
import synth

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def r256(n):
    return (n + 255) // 256 * 256


def make_blob(H, I, gate_codes, up_codes, down_codes, gs, us, ds):
    """Assemble an expert blob from [N][K] nibble codes and [N][K/32] scale bytes."""
    def pack(c):
        c = np.asarray(c, np.uint8)
        return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8).ravel()
    parts = [pack(gate_codes), pack(up_codes), pack(down_codes),
             np.asarray(gs, np.uint8).ravel(), np.asarray(us, np.uint8).ravel(), np.asarray(ds, np.uint8).ravel()]
    out = np.zeros(sum(r256(p.size) for p in parts), np.uint8)
    o = 0
    for p in parts:
        out[o:o + p.size] = p
        o += r256(p.size)
    assert out.size == oracle.expert_bytes(H, I) == synth.expert_bytes(H, I)
    return out


def dec(codes, scales):
    c = np.asarray(codes)
    mag = np.array(E2M1_TABLE)[c & 7]
    return np.where(c & 8, -mag, mag) * np.exp2(np.repeat(np.asarray(scales, np.int64), 32, axis=1) - 127.0)


def bf16_of(v):
    f = np.asarray(v, np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def f64_of(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def _one_hot_expert(rng, H, I, k0, flip_gate=False, zero_gate=False, zero_up=False):
    gc = np.zeros((I, H), np.uint8)
    uc = np.zeros((I, H), np.uint8)
    gc[:, k0] = rng.integers(0, 16, I)
    uc[:, k0] = rng.integers(0, 16, I)
    if zero_gate:
        gc[:] = 0
    if zero_up:
        uc[:] = 0
    if flip_gate:
        gc[:, k0] ^= 8
    dc = rng.integers(0, 16, (H, I)).astype(np.uint8)
    gs = np.full((I, H // 32), 126, np.uint8)
    us = np.full((I, H // 32), 127, np.uint8)
    ds = rng.integers(118, 124, (H, I // 32)).astype(np.uint8)
    return gc, uc, dc, gs, us, ds


def test_routed_expert_one_hot_reduces_to_swiglu_closed_form():
    rng = np.random.default_rng(0)
    H, I, k0 = 64, 32, 37
    gc, uc, dc, gs, us, ds = _one_hot_expert(rng, H, I, k0)
    blob = make_blob(H, I, gc, uc, dc, gs, us, ds)
    x = np.zeros((1, H), np.uint16)
    x[0, k0] = bf16_of(1.0)
    out = oracle.routed_expert(blob, H, I, x)[0]
    g = dec(gc, gs)[:, k0]
    u = dec(uc, us)[:, k0]
    h = (g * expit(g) * u).astype(np.float32).astype(np.float64)
    ref = dec(dc, ds) @ h
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-9)


def test_routed_expert_silu_odd_part_identity():
    """out(g) - out(-g) = W_down (g * u), since silu(z) - silu(-z) = z."""
    rng = np.random.default_rng(1)
    H, I, k0 = 96, 64, 5
    gc, uc, dc, gs, us, ds = _one_hot_expert(rng, H, I, k0)
    x = np.zeros((1, H), np.uint16)
    x[0, k0] = bf16_of(1.0)
    a = oracle.routed_expert(make_blob(H, I, gc, uc, dc, gs, us, ds), H, I, x)[0].astype(np.float64)
    gcf = gc.copy()
    gcf[:, k0] ^= 8
    b = oracle.routed_expert(make_blob(H, I, gcf, uc, dc, gs, us, ds), H, I, x)[0].astype(np.float64)
    g, u = dec(gc, gs)[:, k0], dec(uc, us)[:, k0]
    # a and b are fp32-rounded outputs of magnitude ~|a|: compare with that scale
    assert np.allclose(a - b, dec(dc, ds) @ (g * u), rtol=0, atol=4e-7 * np.abs(a).max())


def test_routed_expert_zero_gate_or_up_gives_zero():
    rng = np.random.default_rng(2)
    H, I = 64, 32
    x = bf16_of(rng.standard_normal((2, H)))
    for kw in ({"zero_gate": True}, {"zero_up": True}):
        blob = make_blob(H, I, *_one_hot_expert(rng, H, I, 3, **kw))
        assert np.all(oracle.routed_expert(blob, H, I, x) == 0)


def test_shared_expert_one_hot_closed_form():
    rng = np.random.default_rng(3)
    H, Is, k0 = 64, 32, 9
    wg = np.zeros((Is, H), np.uint16)
    wu = np.zeros((Is, H), np.uint16)
    wg[:, k0] = bf16_of(rng.standard_normal(Is))
    wu[:, k0] = bf16_of(rng.standard_normal(Is))
    wd = bf16_of(rng.standard_normal((H, Is)) * 0.1)
    x = np.zeros((1, H), np.uint16)
    x[0, k0] = bf16_of(1.0)
    out = oracle.shared_expert(wg, wu, wd, H, Is, x)[0]
    g, u = f64_of(wg[:, k0]), f64_of(wu[:, k0])
    h = (g * expit(g) * u).astype(np.float32).astype(np.float64)
    assert np.allclose(out, f64_of(wd) @ h, rtol=1e-6, atol=1e-9)


def _tiny_layer(seed, E=16, k=2, Is=64, same_expert=False):
    H, I = 256, 64
    rw = synth.fill_bf16(seed, synth.tag(0, synth.KIND_ROUTER), 1.0, E * H).reshape(E, H)
    sg = synth.fill_bf16(seed, synth.tag(0, synth.KIND_SHARED, 0, 0), 0.02, Is * H).reshape(Is, H)
    su = synth.fill_bf16(seed, synth.tag(0, synth.KIND_SHARED, 0, 1), 0.02, Is * H).reshape(Is, H)
    sd = synth.fill_bf16(seed, synth.tag(0, synth.KIND_SHARED, 0, 2), 0.02, H * Is).reshape(H, Is)
    if same_expert:
        b = synth.expert_blob(seed, 0, 0, H, I, 0.02)
        experts = {e: b for e in range(E)}
    else:
        experts = {e: synth.expert_blob(seed, 0, e, H, I, 0.02) for e in range(E)}
    x = synth.fill_bf16(seed, synth.tag(0, synth.KIND_X), 1.0, 3 * H).reshape(3, H)
    res = f64_of(x).astype(np.float32)
    return dict(H=H, I=I, E=E, k=k, Is=Is, router_w=rw, router_bias=None, shared_gate=sg if Is else None,
                shared_up=su if Is else None, shared_down=sd if Is else None, experts=experts, x=x, residual=res)


def _run(L, **over):
    L = {**L, **over}
    return oracle.moe_layer(L["H"], L["I"], L["E"], L["k"], L["Is"], L["router_w"], L["router_bias"],
                            L["shared_gate"], L["shared_up"], L["shared_down"], L["experts"], L["x"],
                            L["residual"], want_stages=True)


def test_layer_identical_experts_gates_drop_out():
    L = _tiny_layer(1, same_expert=True)
    r = _run(L)
    o = oracle.routed_expert(L["experts"][0], 256, 64, L["x"]).astype(np.float64)
    sh = oracle.shared_expert(L["shared_gate"], L["shared_up"], L["shared_down"], 256, 64, L["x"]).astype(np.float64)
    ref = L["residual"].astype(np.float64) + sh + o
    assert np.allclose(r["out"], ref, rtol=1e-6, atol=1e-7)


def test_layer_k_equals_e_is_dense_softmax_mixture():
    L = _tiny_layer(2, k=16)
    r = _run(L)
    lg, _ = oracle.router_logits(L["x"], L["router_w"], None, 256, 16)
    sh = oracle.shared_expert(L["shared_gate"], L["shared_up"], L["shared_down"], 256, 64, L["x"]).astype(np.float64)
    outs = np.stack([oracle.routed_expert(L["experts"][e], 256, 64, L["x"]) for e in range(16)], 1).astype(np.float64)
    for b in range(3):
        p = softmax(lg[b].astype(np.float64))
        ref = L["residual"][b].astype(np.float64) + sh[b] + p @ outs[b]
        assert np.allclose(r["out"][b], ref, rtol=1e-6, atol=1e-6)


def test_layer_stages_and_residual_and_no_shared():
    L = _tiny_layer(3)
    r = _run(L)
    # every slot equals its expert applied to its row
    for b in range(3):
        assert len(set(r["idx"][b].tolist())) == 2
        for j in range(2):
            e = int(r["idx"][b, j])
            assert np.array_equal(r["slots"][b, j], oracle.routed_expert(L["experts"][e], 256, 64, L["x"][b:b + 1])[0])
    # residual enters additively
    r2 = _run(L, residual=L["residual"] + np.float32(8.0))
    assert np.allclose(r2["out"] - r["out"], 8.0, atol=2e-6)
    # no shared expert: out = residual + sum_j g_j o_j
    r3 = _run(L, Is=0, shared_gate=None, shared_up=None, shared_down=None)
    ref = L["residual"].astype(np.float64) + np.einsum("bj,bjh->bh", r["gate"].astype(np.float64),
                                                      r["slots"].astype(np.float64))
    assert np.allclose(r3["out"], ref, rtol=1e-6, atol=1e-7)


def test_layer_same_result_on_one_or_many_threads():
    """The layer's expert evaluations may run on several host threads: the
    result is bit-identical to one thread's."""
    L = _tiny_layer(5)
    n0 = oracle.set_threads(0)
    try:
        oracle.set_threads(1)
        r1 = _run(L)
        oracle.set_threads(max(2, n0))
        rn = _run(L)
    finally:
        oracle.set_threads(n0)
    for key in ("out", "idx", "gate", "shared", "slots"):
        assert np.array_equal(r1[key].view(np.uint8), rn[key].view(np.uint8)), key


def test_layer_missing_expert_blob_is_an_error():
    L = _tiny_layer(4)
    with pytest.raises(ValueError):
        _run(L, experts={})


# ---- dense-block pieces --------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        ((rng.integers(0, 2 ** 16, 4000).astype(np.uint32) << 16) | 0x8000).view(np.float32),  # exact ties
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38], np.float32),
    ])
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.to_bf16(v), ref)


def test_rmsnorm_closed_forms():
    h = np.full((1, 64), -3.0, np.float32)
    assert np.all(oracle.rmsnorm_bf16(h, eps=0.0) == 0xBF80)  # -1.0
    one = np.zeros((1, 4), np.float32)
    one[0, 2] = 5.0
    out = oracle.rmsnorm_bf16(one, eps=0.0)
    assert out[0].tolist() == [0, 0, 0x4000, 0]  # 5 / sqrt(25/4) = 2
    rng = np.random.default_rng(6)
    hh = rng.standard_normal((3, 256)).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm_bf16(hh, 0.0), oracle.rmsnorm_bf16(hh * 4, 0.0))
    # eps enters under the root: all-ones with eps 3 -> 1/2
    assert np.all(oracle.rmsnorm_bf16(np.ones((1, 8), np.float32), eps=3.0) == 0x3F00)


def test_dense_gemv_permutation_and_sum():
    rng = np.random.default_rng(7)
    K = 128
    perm = rng.permutation(K)
    w = np.zeros((K, K), np.uint16)
    w[np.arange(K), perm] = bf16_of(1.0)
    x = bf16_of(rng.standard_normal((2, K)))
    assert np.array_equal(oracle.dense_gemv_bf16(w, x), x[:, perm])
    ones = np.full((1, K), bf16_of(1.0), np.uint16)
    y = oracle.dense_gemv_bf16(ones, x)
    for b in range(2):
        s = np.float32(math.fsum(f64_of(x[b])))
        assert y[b, 0] == oracle.to_bf16(np.array([s]))[0]
