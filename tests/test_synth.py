"""Host-side checks of the seeded input generator (no GPU).

The generator is input preparation only; these tests pin its published
building blocks (SplitMix64 finaliser, Irwin-Hall normal, bf16 rounding,
MXFP4 encoding rules of OCP MX v1.0) and its determinism.  Byte equality of
the host and device builds is checked in tests/test_gpu_synth.py.
"""
import math

import numpy as np
import torch

import oracle
import synth

M64 = 0xFFFFFFFFFFFFFFFF


def mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix64_sequence():
    # SplitMix64 as a sequential generator: state += GAMMA; out = mix64(state).
    # The counter form draw(key, i) = mix64(key + (i+1) GAMMA) is the same stream.
    seed, t = 12345, synth.tag(1, synth.KIND_EXPERT, 7, 2)
    k = synth.key(seed, t)
    state = k
    for i in range(50):
        state = (state + 0x9E3779B97F4A7C15) & M64
        assert synth.draw(seed, t, i) == mix64(state)


def test_gauss_int_is_irwin_hall_of_8_fields():
    seed, t = 3, synth.tag(0, synth.KIND_X)
    for i in range(100):
        a, b = synth.draw(seed, t, 2 * i), synth.draw(seed, t, 2 * i + 1)
        s = sum((a >> (16 * j)) & 0xFFFF for j in range(4)) + sum((b >> (16 * j)) & 0xFFFF for j in range(4))
        assert synth.gauss_int(seed, t, i) == 2 * s - 8 * 65535


def test_normal_moments():
    v = synth.fill_f32(9, synth.tag(0, synth.KIND_H0), 1.0, 4_000_000).astype(np.float64)
    assert abs(v.mean()) < 3e-3
    assert abs(v.std() - 1.0) < 3e-3
    assert abs(np.mean(v ** 4) / np.mean(v ** 2) ** 2 - 2.85) < 0.05  # Irwin-Hall(8) kurtosis = 3 - 1.2/8
    w = synth.fill_f32(9, synth.tag(0, synth.KIND_ROUTER), 0.02, 1_000_000).astype(np.float64)
    assert abs(w.std() - 0.02) < 1e-4


def test_bf16_fill_is_rne_of_f32_fill():
    n = 100_000
    t = synth.tag(2, synth.KIND_DENSE, 0, 3)
    f = synth.fill_f32(5, t, 0.02, n)
    b = synth.fill_bf16(5, t, 0.02, n)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
    rows = synth.bf16_rows(5, t, 0.02, 1000, 10, 20)
    assert np.array_equal(rows.ravel(), b[10_000:30_000])


def test_quantiser_rules():
    # scale choice: floor(log2(amax)) - 2
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 6.0 * 2.0 ** -8
    codes, scales = synth.quantise(w)
    assert scales[0, 0] == 127 - 8 and codes[0, 0] == 7
    # all zero block: scale 127, codes 0
    codes, scales = synth.quantise(np.zeros((1, 32), np.float32))
    assert scales[0, 0] == 127 and not codes.any()
    # ties to even on the E2M1 grid and saturation at 6 (scale fixed by a 4.0 entry)
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9, 0.3, -0.75]
    expect = [0, 2, 2, 4, 4, 6, 6, 7, 1, 10]
    w = np.zeros((1, 32), np.float32)
    w[0, :len(vals)] = vals
    w[0, 31] = 4.0
    codes, scales = synth.quantise(w)
    assert scales[0, 0] == 127
    nib = np.stack([codes[0] & 15, codes[0] >> 4], 1).ravel()
    assert nib[:len(vals)].tolist() == expect
    # random blocks: decoded value is the nearest grid point
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    codes, scales = synth.quantise(w)
    d = oracle.decode_mxfp4(codes, scales, 64, 256).astype(np.float64)
    step = np.exp2(np.repeat(scales.astype(np.int64), 32, 1) - 127.0)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    a = np.minimum(np.abs(w) / step, 6.0)
    best = np.abs(a[..., None] - grid).min(-1)
    assert np.allclose(np.abs(np.abs(d) / step - a), best, atol=1e-6)
    assert 0xFF not in scales


def test_expert_blob_layout_and_determinism():
    H, I = 256, 64
    assert synth.expert_bytes(7168, 1536) == 17547264
    for H_, I_ in ((32, 32), (96, 64), (256, 64), (7168, 1536), (4096, 352)):
        assert synth.expert_bytes(H_, I_) == oracle.expert_bytes(H_, I_)
    b1 = synth.expert_blob(7, 0, 3, H, I, 0.02)
    b2 = synth.expert_blob(7, 0, 3, H, I, 0.02)
    b3 = synth.expert_blob(7, 0, 4, H, I, 0.02)
    assert np.array_equal(b1, b2) and not np.array_equal(b1, b3)
    off = synth.expert_offsets(H, I)
    # gate matrix = quantised N(0, 0.02) samples of the expert's gate stream
    t = synth.tag(0, synth.KIND_EXPERT, 3, 0)
    g = synth.fill_f32(7, t, 0.02, I * H).reshape(I, H)
    codes, scales = synth.quantise(g)
    assert np.array_equal(b1[off[0]:off[0] + I * H // 2], codes.ravel())
    assert np.array_equal(b1[off[3]:off[3] + I * H // 32], scales.ravel())


def test_zipf_bias_is_log_rank():
    b = synth.zipf_bias(0, 0, 896, 1.1)
    ranks = np.exp(-b.astype(np.float64) / 1.1)
    assert np.allclose(np.sort(ranks), np.arange(1, 897), rtol=1e-5)
    assert not np.array_equal(b, synth.zipf_bias(1, 0, 896, 1.1))
