"""Pins of the oracle's MXFP8 activation quantisation (the FP4 x MXFP8 expert
variant of "Kimi K3 on GB300: 13 kernels a layer, and what 842 and 423 tokens
a second measure", section "Why batch 1 on a rack is not only a bandwidth
problem").

What pins it: every E4M3 code against torch's float8_e4m3fn (an independent
implementation of the OCP 8-bit format) and the format's named extremes;
element rounding against torch's round-to-nearest-even conversion on blocks
whose shared scale is 1; saturation at 448; the shared scale by the property
that defines it (each block's largest magnitude lands in [256, 512) times the
scale, the top binade of E4M3); values already on the grid round-tripping
exactly; the half-ulp error bound; and the expert variant against a one-hot
closed form built from those pinned pieces.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from test_oracle_layer import _one_hot_expert, bf16_of, dec, make_blob


def test_all_e4m3_codes_match_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 is code 0x80


def test_e4m3_named_values():
    assert oracle.e4m3(0x7E) == 448.0              # largest finite magnitude, 1.75 * 2^8
    assert oracle.e4m3(0x08) == 2.0 ** -6          # smallest normal
    assert oracle.e4m3(0x07) == 0.875 * 2.0 ** -6  # largest subnormal
    assert oracle.e4m3(0x01) == 2.0 ** -9          # smallest subnormal
    assert oracle.e4m3(0x38) == 1.0 and oracle.e4m3(0xC0) == -2.0


def _blocks_with_unit_scale(rng, nblocks):
    """Blocks whose largest magnitude is in [256, 448]: the shared scale is 2^0."""
    v = rng.uniform(-448, 448, (nblocks, 32))
    v[:, 0] = rng.uniform(256, 448, nblocks) * rng.choice([-1, 1], nblocks)
    v[:, 1:] = np.clip(v[:, 1:], -np.abs(v[:, :1]), np.abs(v[:, :1]))
    # exact ties between neighbouring E4M3 values and tiny / subnormal values
    v[:, 2] = (np.floor(rng.uniform(8, 15, nblocks)) + 0.5) * 2.0 ** -3       # ties at spacing 1/8
    v[:, 3] = rng.uniform(-2.0 ** -6, 2.0 ** -6, nblocks)                      # subnormal range
    v[:, 4] = (np.floor(rng.uniform(0, 7, nblocks)) + 0.5) * 2.0 ** -9          # subnormal ties
    return v.astype(np.float32)


def test_element_rounding_matches_torch_rne_where_the_scale_is_one():
    rng = np.random.default_rng(0)
    v = _blocks_with_unit_scale(rng, 400)
    codes, scales = oracle.quantize_mxfp8(v)
    assert np.all(scales == 127)
    ref = torch.from_numpy(v.ravel()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_magnitudes_past_448_saturate():
    v = np.zeros(32, np.float32)
    v[:6] = [464.0, -470.0, 479.9, 500.0, -511.0, 300.0]  # block max < 512: scale 2^0
    codes, scales = oracle.quantize_mxfp8(v)
    assert scales[0] == 127
    assert list(codes[:6]) == [0x7E, 0xFE, 0x7E, 0x7E, 0xFE, 0x79]  # 300 -> 288 (1.125 * 2^8)


def test_shared_scale_puts_each_block_max_in_the_top_binade():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((300, 32)) * np.exp2(rng.integers(-30, 30, (300, 1)))).astype(np.float32)
    codes, scales = oracle.quantize_mxfp8(v)
    X = np.exp2(scales.astype(np.float64) - 127.0)
    amax = np.abs(v.astype(np.float64)).max(axis=1)
    assert np.all(amax / X >= 256.0) and np.all(amax / X < 512.0)


def test_zero_block_and_grid_round_trip():
    codes, scales = oracle.quantize_mxfp8(np.zeros(32, np.float32))
    assert scales[0] == 0 and np.all(codes == 0)
    rng = np.random.default_rng(2)
    # values on the grid: E4M3 finite codes times 2^k, with a top-binade block max
    finite = [c for c in range(0x7F) if c != 0]
    for k in (-20, -3, 0, 5):
        c = rng.choice(finite, 32)
        c[0] = 0x78 + rng.integers(0, 7)  # magnitude in [256, 448]
        sign = rng.choice([0, 0x80], 32)
        v = np.array([oracle.e4m3(int(ci | si)) for ci, si in zip(c, sign)]) * 2.0 ** k
        q, s = oracle.quantize_mxfp8(v.astype(np.float32))
        assert s[0] == 127 + k
        assert np.array_equal(oracle.dequantize_mxfp8(q, s), v.astype(np.float32))


def test_quantisation_error_within_half_an_ulp():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((500, 32)).astype(np.float32)
    q, s = oracle.quantize_mxfp8(v)
    d = oracle.dequantize_mxfp8(q, s).reshape(v.shape).astype(np.float64)
    X = np.exp2(s.astype(np.float64) - 127.0)[:, None]
    a = np.abs(v.astype(np.float64))
    # normal range of E4M3 (>= 2^-6 X): 3 mantissa bits, so half an ulp is <= 2^-4 of the value;
    # below it the spacing is 2^-9 X; above 448 X (a block max can reach 512 X) it saturates to 448 X
    bound = np.where(a >= 2.0 ** -6 * X, 2.0 ** -4 * a, 2.0 ** -10 * X)
    bound = np.maximum(bound, a - 448.0 * X)
    assert np.all(np.abs(d - v) <= bound * (1 + 1e-12))


def test_mx8_expert_on_a_one_hot_row_is_fc2_of_the_quantised_swiglu():
    """x one-hot (1.0, exactly representable in MXFP8): FC1 reads one decoded
    column as in the exact expert; FC2 then runs on the MXFP8 quantisation of
    h = silu(g) * u."""
    rng = np.random.default_rng(4)
    H, I, k0 = 64, 32, 37
    gc, uc, dc, gs, us, ds = _one_hot_expert(rng, H, I, k0)
    blob = make_blob(H, I, gc, uc, dc, gs, us, ds)
    x = np.zeros((1, H), np.uint16)
    x[0, k0] = bf16_of(1.0)
    out = oracle.routed_expert(blob, H, I, x, mx8=True)[0]
    g = dec(gc, gs)[:, k0]
    u = dec(uc, us)[:, k0]
    h = (g * expit(g) * u).astype(np.float32)
    hq = oracle.dequantize_mxfp8(*oracle.quantize_mxfp8(h)).astype(np.float64)
    ref = dec(dc, ds) @ hq
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-9)
    exact = oracle.routed_expert(blob, H, I, x)[0]
    assert not np.array_equal(out, exact)  # h is not on the MXFP8 grid: the variant differs


@pytest.mark.parametrize("seed", [0, 1])
def test_mx8_layer_close_to_the_exact_layer(seed):
    """The variant's layer output stays within a few percent of the exact one
    (E4M3 keeps 4 significant bits: ~2^-5 relative rms error per element,
    averaged down over the dot products)."""
    from test_oracle_layer import _run, _tiny_layer
    L = _tiny_layer(seed)
    a = _run(L)
    b = oracle.moe_layer(L["H"], L["I"], L["E"], L["k"], L["Is"], L["router_w"], L["router_bias"],
                         L["shared_gate"], L["shared_up"], L["shared_down"], L["experts"], L["x"], L["residual"],
                         want_stages=True, mx8=True)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["shared"], b["shared"])
    d = b["slots"].astype(np.float64) - a["slots"]
    rel = np.linalg.norm(d.reshape(-1, L["H"]), axis=1) / np.linalg.norm(a["slots"].reshape(-1, L["H"]), axis=1)
    assert 1e-3 < rel.max() < 0.1
