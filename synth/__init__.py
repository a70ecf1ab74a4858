"""Seeded synthetic inputs for the MXFP4 MoE decode layer.

This module is the only code the CPU oracle and the GPU library have in
common, and it holds none of the layer's arithmetic (see ``synth_core.h``).
Two builds of the same counter-based generator exist:

* ``libsynth_host.so`` (gcc + OpenMP) regenerates any tensor, or any single
  expert, on the host -- the oracle's inputs;
* ``libsynth_dev.so`` (hipcc, gfx950) writes the same bytes straight into
  HBM -- the GPU path's inputs -- so a layer's 15.7 GB of MXFP4 experts is
  made on the device in milliseconds instead of being copied over PCIe.

``tests/test_synth.py`` checks the host build against its definition and
``tests/test_gpu_synth.py`` checks that both builds agree byte for byte.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, LayerConfig  # noqa: F401

_DIR = os.path.dirname(os.path.abspath(__file__))
_HOST_SO = os.path.join(_DIR, "libsynth_host.so")
_DEV_SO = os.path.join(_DIR, "libsynth_dev.so")
_host = None
_dev = None

KIND_X, KIND_ROUTER, KIND_BIASPERM, KIND_SHARED, KIND_EXPERT, KIND_DENSE, KIND_H0 = 1, 2, 3, 4, 5, 6, 7

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host() -> str:
    tmp = _HOST_SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                           os.path.join(_DIR, "synth_host.c"), "-o", tmp, "-lm"])
    os.replace(tmp, _HOST_SO)
    return _HOST_SO


def build_dev() -> str:
    tmp = _DEV_SO + ".tmp"
    subprocess.check_call([HIPCC, *HIP_FLAGS, os.path.join(_DIR, "synth_dev.hip"), "-o", tmp],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, _DEV_SO)
    return _DEV_SO


def build() -> None:
    build_host()
    build_dev()


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(_HOST_SO):
            build_host()
        lib = ctypes.CDLL(_HOST_SO)
        U64, U32, D, P, F = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p, ctypes.c_float
        sig = {
            "synth_mult": (F, [D]),
            "synth_tag": (U64, [U32, U32, U32, U32]),
            "synth_draw": (U64, [U64, U64, U64]),
            "synth_gauss_int": (ctypes.c_int32, [U64, U64, U64]),
            "synth_fill_f32": (None, [U64, U64, D, P, U64]),
            "synth_fill_bf16": (None, [U64, U64, D, P, U64]),
            "synth_fill_bf16_rows": (None, [U64, U64, D, U64, U64, U64, P]),
            "synth_expert_bytes": (U64, [U64, U64]),
            "synth_expert_offsets": (None, [U64, U64, P]),
            "synth_expert_blob": (None, [U64, U32, U32, U64, U64, D, P]),
            "synth_quantise": (None, [P, U64, U64, P, P]),
            "synth_zipf_bias": (None, [U64, U32, U32, D, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_SO):
            build_dev()
        lib = ctypes.CDLL(_DEV_SO)
        U64, U32, P, F, I = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        lib.synth_dev_fill_bf16.restype = I
        lib.synth_dev_fill_bf16.argtypes = [U64, F, P, U64, P]
        lib.synth_dev_fill_f32.restype = I
        lib.synth_dev_fill_f32.argtypes = [U64, F, P, U64, P]
        lib.synth_dev_expert_blobs.restype = I
        lib.synth_dev_expert_blobs.argtypes = [U64, U32, U32, U32, U64, U64, F, P, U64, P]
        _dev = lib
    return _dev


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- host side ----------------------------------------------------------------

def tag(layer: int, kind: int, expert: int = 0, matrix: int = 0) -> int:
    return int(_host_lib().synth_tag(layer, kind, expert, matrix))


def mult(sigma: float) -> float:
    return float(_host_lib().synth_mult(sigma))


def key(seed: int, t: int) -> int:
    """key(seed, tag) = mix64(seed * GAMMA + tag) (mod 2^64)."""
    g = 0x9E3779B97F4A7C15
    z = (seed * g + t) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return z ^ (z >> 31)


def draw(seed: int, t: int, i: int) -> int:
    return int(_host_lib().synth_draw(seed, t, i))


def gauss_int(seed: int, t: int, i: int) -> int:
    return int(_host_lib().synth_gauss_int(seed, t, i))


def fill_f32(seed: int, t: int, sigma: float, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    _host_lib().synth_fill_f32(seed, t, sigma, _ptr(out), n)
    return out


def fill_bf16(seed: int, t: int, sigma: float, n: int) -> np.ndarray:
    out = np.empty(n, np.uint16)
    _host_lib().synth_fill_bf16(seed, t, sigma, _ptr(out), n)
    return out


def bf16_rows(seed: int, t: int, sigma: float, K: int, r0: int, nr: int) -> np.ndarray:
    out = np.empty((nr, K), np.uint16)
    _host_lib().synth_fill_bf16_rows(seed, t, sigma, K, r0, nr, _ptr(out))
    return out


def expert_bytes(H: int, I: int) -> int:
    return int(_host_lib().synth_expert_bytes(H, I))


def expert_offsets(H: int, I: int) -> list:
    off = np.zeros(6, np.uint64)
    _host_lib().synth_expert_offsets(H, I, _ptr(off))
    return [int(v) for v in off]


def expert_blob(seed: int, layer: int, expert: int, H: int, I: int, sigma: float) -> np.ndarray:
    out = np.empty(expert_bytes(H, I), np.uint8)
    _host_lib().synth_expert_blob(seed, layer, expert, H, I, sigma, _ptr(out))
    return out


def quantise(w: np.ndarray):
    """MXFP4-encode an fp32 [N][K] matrix with the generator's encoder -> (codes, scales)."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    _host_lib().synth_quantise(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def zipf_bias(seed: int, layer: int, E: int, s: float) -> np.ndarray:
    out = np.empty(E, np.float32)
    _host_lib().synth_zipf_bias(seed, layer, E, s, _ptr(out))
    return out


# ---- device side (torch tensors in HBM) ----------------------------------------

def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def dev_fill_bf16(out, seed: int, t: int, sigma: float, stream=0):
    """Fill a contiguous int16/bfloat16 CUDA tensor with bf16 samples (element index = flat index)."""
    _check(_dev_lib().synth_dev_fill_bf16(key(seed, t), mult(sigma), out.data_ptr(), out.numel(), stream),
           "synth_dev_fill_bf16")


def dev_fill_f32(out, seed: int, t: int, sigma: float, stream=0):
    _check(_dev_lib().synth_dev_fill_f32(key(seed, t), mult(sigma), out.data_ptr(), out.numel(), stream),
           "synth_dev_fill_f32")


def dev_expert_blobs(out, seed: int, layer: int, e0: int, ne: int, H: int, I: int, sigma: float, stream=0):
    """Write experts e0..e0+ne-1 into a zeroed uint8 CUDA tensor of ne * expert_bytes(H, I) bytes."""
    nb = expert_bytes(H, I)
    if out.numel() < ne * nb:
        raise ValueError("expert buffer too small")
    _check(_dev_lib().synth_dev_expert_blobs(seed, layer, e0, ne, H, I, mult(sigma), out.data_ptr(), nb, stream),
           "synth_dev_expert_blobs")
