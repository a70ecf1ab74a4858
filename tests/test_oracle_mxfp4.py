"""Pins of the oracle's MXFP4 decode and GEMV against the format definition,
the pages' printed expert size, closed forms and brute force.

The E2M1 value table and the E8M0 scale rule are those printed in the OCP
Microscaling Formats (MX) v1.0 specification (tables of the FP4 E2M1 and
E8M0 formats); the 17,547,264-byte expert size is from "Kimi K3 on GB300: 13
kernels a layer" (section "What one decode step of Kimi K3 does").
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")

# OCP MX v1.0, FP4 (E2M1) table: magnitudes of codes 0..7; codes 8..15 are the negatives.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def pack(codes_2d):
    """[N][K] nibble codes -> [N][K/2] bytes, element 2i in bits 3:0, 2i+1 in 7:4."""
    c = np.asarray(codes_2d, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def table_decode(codes_2d, scales_2d):
    c = np.asarray(codes_2d)
    mag = np.array(E2M1_TABLE)[c & 7]
    val = np.where(c & 8, -mag, mag)
    sc = np.repeat(np.asarray(scales_2d, np.int64), 32, axis=1)
    return val * np.exp2(sc - 127.0)


def test_e2m1_all_16_codes():
    for c in range(16):
        v = oracle.e2m1(c)
        exp = E2M1_TABLE[c & 7] * (-1 if c & 8 else 1)
        assert v == exp, (c, v, exp)
    assert math.copysign(1.0, oracle.e2m1(8)) == -1.0  # code 8 is -0


def test_e8m0_scales_roundtrip_and_nan():
    for e in range(255):
        v = oracle.e8m0(e)
        m, ex = math.frexp(v)
        assert m == 0.5  # a pure power of two
        assert ex - 1 + 127 == e  # encode(decode(e)) == e
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(0) == 2.0 ** -127
    assert math.isnan(oracle.e8m0(255))


def test_expert_bytes_matches_pages():
    g = json.load(open(GOLDEN))["expert_bytes_k3"]
    assert oracle.expert_bytes(g["hidden"], g["inter"]) == g["value"]
    # 896 experts of a layer; 1,472 experts a token = 25.83 GB
    assert 896 * g["value"] == 15_722_348_544
    t = json.load(open(GOLDEN))["experts_per_token"]
    assert t["layers_moe"] * t["top_k"] == t["experts"]
    assert round(t["experts"] * g["value"] / 1e9, 2) == t["gigabytes"]
    # the tiny workload: 3 x 8192 code bytes + 3 x 512 scale bytes
    assert oracle.expert_bytes(256, 64) == 26112


def test_decode_one_hot_positions_and_nibble_order():
    N, K = 3, 64
    rng = np.random.default_rng(0)
    for n in range(N):
        for k in (0, 1, 30, 31, 32, 33, 63):
            codes = np.zeros((N, K), np.uint8)
            code = int(rng.integers(1, 16))
            if code == 8:
                code = 9
            codes[n, k] = code
            scales = np.full((N, K // 32), 127, np.uint8)
            scales[n, k // 32] = 125
            w = oracle.decode_mxfp4(pack(codes), scales, N, K)
            exp = np.zeros((N, K))
            exp[n, k] = E2M1_TABLE[code & 7] * (-1 if code & 8 else 1) * 0.25
            assert np.array_equal(w, exp), (n, k, code)


def test_decode_matches_table_random():
    rng = np.random.default_rng(1)
    N, K = 5, 96
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = rng.integers(0, 255, (N, K // 32)).astype(np.uint8)
    w = oracle.decode_mxfp4(pack(codes), scales, N, K)
    assert np.array_equal(w.astype(np.float64), table_decode(codes, scales))


def _bf16(x):
    """float64 -> bf16 bits via float32 truncation of exactly-representable values."""
    f = np.asarray(x, np.float32)
    assert np.all((f.view(np.uint32) & 0xFFFF) == 0)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_to_f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_gemv_all_ones_is_sum_of_x():
    rng = np.random.default_rng(2)
    N, K = 4, 256
    codes = pack(np.full((N, K), 2, np.uint8))  # code 2 = 1.0
    scales = np.full((N, K // 32), 127, np.uint8)
    x = _rand_bf16(rng, (3, K))
    y = oracle.gemv_mxfp4(codes, scales, N, K, x)
    for b in range(3):
        s = np.float32(math.fsum(_bf16_to_f64(x[b])))
        assert np.all(y[b] == s)


def test_gemv_one_hot_x_gives_decoded_column():
    rng = np.random.default_rng(3)
    N, K = 6, 128
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    dec = table_decode(codes, scales)
    for k in (0, 1, 2, 63, 64, 127):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = _bf16(1.0)
        y = oracle.gemv_mxfp4(pack(codes), scales, N, K, x)
        assert np.array_equal(y[0].astype(np.float64), dec[:, k])


def test_gemv_scale_and_sign_symmetries():
    rng = np.random.default_rng(4)
    N, K = 8, 192
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = rng.integers(115, 125, (N, K // 32)).astype(np.uint8)
    x = _rand_bf16(rng, (2, K))
    y = oracle.gemv_mxfp4(pack(codes), scales, N, K, x)
    y2 = oracle.gemv_mxfp4(pack(codes), scales + 1, N, K, x)
    assert np.array_equal(y2, 2 * y)
    yneg = oracle.gemv_mxfp4(pack(codes ^ 8), scales, N, K, x)
    assert np.array_equal(yneg, -y)


def test_gemv_nan_scale_poisons_exactly_its_rows():
    rng = np.random.default_rng(5)
    N, K = 5, 96
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = np.full((N, K // 32), 127, np.uint8)
    scales[2, 1] = 255
    x = _rand_bf16(rng, (2, K))
    y = oracle.gemv_mxfp4(pack(codes), scales, N, K, x)
    assert np.all(np.isnan(y[:, 2]))
    assert not np.any(np.isnan(np.delete(y, 2, axis=1)))


def test_gemv_brute_force_matches_library_matmul():
    rng = np.random.default_rng(6)
    for N, K in ((7, 32), (16, 256), (3, 1536)):
        codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
        scales = rng.integers(118, 124, (N, K // 32)).astype(np.uint8)
        dec = table_decode(codes, scales)
        xb = _rand_bf16(rng, (3, K))
        xf = rng.standard_normal((2, K)).astype(np.float32)
        yb = oracle.gemv_mxfp4(pack(codes), scales, N, K, xb)
        yf = oracle.gemv_mxfp4(pack(codes), scales, N, K, xf)
        ref_b = _bf16_to_f64(xb) @ dec.T
        ref_f = xf.astype(np.float64) @ dec.T
        # the oracle rounds a double sum to fp32 once: within 1 fp32 ulp of the
        # library's double result (plus the double rounding noise)
        assert np.allclose(yb, ref_b, rtol=2 ** -23, atol=1e-30 + np.abs(ref_b).max() * 1e-15)
        assert np.allclose(yf, ref_f, rtol=2 ** -23, atol=1e-30 + np.abs(ref_f).max() * 1e-15)


def test_generator_quantiser_roundtrip_through_oracle_decode():
    """Values on the E2M1 x 2^s grid survive the generator's encoder and the
    oracle's decoder unchanged (the encoder is input preparation; this pins
    that both use the same layout convention)."""
    import synth
    rng = np.random.default_rng(7)
    N, K = 4, 64
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    codes[:, ::32] = 7  # block amax = 6 * scale, so the encoder picks this scale
    scales = rng.integers(100, 140, (N, K // 32)).astype(np.uint8)
    w = table_decode(codes, scales).astype(np.float32)
    c2, s2 = synth.quantise(w)
    assert np.array_equal(s2, scales)
    assert np.array_equal(oracle.decode_mxfp4(c2, s2, N, K), w)
