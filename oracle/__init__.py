"""CPU oracle of the MXFP4 MoE decode layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, and a missing GPU
library is never replaced by it.

The C++ source (``oracle.cpp``) computes every stage from its definition
with double accumulation; this module is a thin ctypes binding that takes
and returns numpy arrays.  Its functions are pinned against closed forms,
printed tables and brute force in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_DIR, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.cpp into liboracle.so (plain g++; OpenMP spreads a layer's
    independent expert evaluations over host threads)."""
    src = os.path.join(_DIR, "oracle.cpp")
    tmp = _SO + ".tmp"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", "-fopenmp", src, "-o", tmp])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    P, I, U64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_double
    sig = {
        "oracle_e2m1": (D, [I]),
        "oracle_e8m0": (D, [I]),
        "oracle_expert_bytes": (U64, [I, I]),
        "oracle_decode_mxfp4": (None, [P, P, I, I, P]),
        "oracle_gemv_mxfp4": (None, [P, P, I, I, P, I, I, P]),
        "oracle_router_logits": (I, [P, P, P, I, I, I, P]),
        "oracle_topk": (None, [P, I, I, I, P, P]),
        "oracle_shared_expert": (None, [P, P, P, I, I, P, I, P]),
        "oracle_routed_expert": (None, [P, I, I, P, I, P]),
        "oracle_moe_layer": (I, [I, I, I, I, I, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P]),
        "oracle_to_bf16": (None, [P, U64, P]),
        "oracle_rmsnorm_bf16": (None, [P, I, I, D, P]),
        "oracle_dense_gemv_bf16": (None, [P, I, I, P, I, P]),
        "oracle_set_threads": (I, [I]),
        "oracle_e4m3": (D, [I]),
        "oracle_quantize_mxfp8": (None, [P, I, P, P]),
        "oracle_dequantize_mxfp8": (None, [P, P, I, P]),
        "oracle_routed_expert_ex": (None, [P, I, I, P, I, P, I]),
        "oracle_moe_layer_ex": (I, [I, I, I, I, I, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e2m1(code: int) -> float:
    return _load().oracle_e2m1(int(code))


def e8m0(byte: int) -> float:
    return _load().oracle_e8m0(int(byte))


def expert_bytes(H: int, I: int) -> int:
    return int(_load().oracle_expert_bytes(H, I))


def decode_mxfp4(codes, scales, N, K):
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    w = np.empty((N, K), np.float32)
    _load().oracle_decode_mxfp4(_p(codes), _p(scales), N, K, _p(w))
    return w


def gemv_mxfp4(codes, scales, N, K, x):
    """y[b][n] = fp32(sum_k w[n][k] x[b][k]); x is bf16 bits (uint16) or float32 [B][K]."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    x_f32 = 1 if x.dtype == np.float32 else 0
    x = _c(x, np.float32 if x_f32 else np.uint16).reshape(-1, K)
    y = np.empty((x.shape[0], N), np.float32)
    _load().oracle_gemv_mxfp4(_p(codes), _p(scales), N, K, _p(x), x_f32, x.shape[0], _p(y))
    return y


def router_logits(x, wr, bias, H, E):
    """Returns (logits fp32 [B][E], number of order-dependent double sums)."""
    x = _c(x, np.uint16).reshape(-1, H)
    wr = _c(wr, np.uint16)
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((x.shape[0], E), np.float32)
    od = _load().oracle_router_logits(_p(x), _p(wr), _p(b), x.shape[0], H, E, _p(out))
    return out, od


def topk(logits, k):
    logits = _c(logits, np.float32)
    B, E = logits.shape
    idx = np.empty((B, k), np.int32)
    gate = np.empty((B, k), np.float32)
    _load().oracle_topk(_p(logits), B, E, k, _p(idx), _p(gate))
    return idx, gate


def shared_expert(wg, wu, wd, H, Is, x):
    x = _c(x, np.uint16).reshape(-1, H)
    out = np.empty((x.shape[0], H), np.float32)
    _load().oracle_shared_expert(_p(_c(wg, np.uint16)), _p(_c(wu, np.uint16)), _p(_c(wd, np.uint16)), H, Is,
                                 _p(x), x.shape[0], _p(out))
    return out


def routed_expert(blob, H, I, x, mx8=False):
    """One routed MXFP4 expert on rows x (bf16 bits); mx8: the FP4 x MXFP8 variant."""
    x = _c(x, np.uint16).reshape(-1, H)
    out = np.empty((x.shape[0], H), np.float32)
    _load().oracle_routed_expert_ex(_p(_c(blob, np.uint8)), H, I, _p(x), x.shape[0], _p(out), int(bool(mx8)))
    return out


def e4m3(code: int) -> float:
    return _load().oracle_e4m3(int(code))


def quantize_mxfp8(v):
    """MXFP8 quantisation of float32 values (length a multiple of 32): (codes uint8, scales uint8)."""
    v = _c(v, np.float32).ravel()
    codes = np.empty(v.size, np.uint8)
    scales = np.empty(v.size // 32, np.uint8)
    _load().oracle_quantize_mxfp8(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def dequantize_mxfp8(codes, scales):
    codes, scales = _c(codes, np.uint8).ravel(), _c(scales, np.uint8).ravel()
    v = np.empty(codes.size, np.float32)
    _load().oracle_dequantize_mxfp8(_p(codes), _p(scales), codes.size, _p(v))
    return v


def moe_layer(H, I, E, k, Is, router_w, router_bias, shared_gate, shared_up, shared_down, experts, x, residual,
              want_stages=False, mx8=False):
    """experts: mapping expert id -> uint8 blob (only selected experts are needed).
    mx8: the routed experts run the FP4 x MXFP8 variant.

    Returns dict(out, idx, gate, order_dependent[, logits, shared, slots]).
    """
    x = _c(x, np.uint16).reshape(-1, H)
    B = x.shape[0]
    residual = _c(residual, np.float32).reshape(B, H)
    keep = {e: _c(b, np.uint8) for e, b in experts.items()}
    table = (ctypes.c_void_p * E)()
    for e, b in keep.items():
        table[e] = b.ctypes.data
    out = np.empty((B, H), np.float32)
    idx = np.empty((B, k), np.int32)
    gate = np.empty((B, k), np.float32)
    logits = np.empty((B, E), np.float32) if want_stages else None
    shared = np.empty((B, H), np.float32) if want_stages else None
    slots = np.empty((B, k, H), np.float32) if want_stages else None
    rw = _c(router_w, np.uint16)
    rb = None if router_bias is None else _c(router_bias, np.float32)
    sg = None if shared_gate is None else _c(shared_gate, np.uint16)
    su = None if shared_up is None else _c(shared_up, np.uint16)
    sd = None if shared_down is None else _c(shared_down, np.uint16)
    rc = _load().oracle_moe_layer_ex(H, I, E, k, Is, _p(rw), _p(rb), _p(sg), _p(su), _p(sd),
                                     ctypes.cast(table, ctypes.c_void_p), _p(x), _p(residual), B, _p(out), _p(idx),
                                     _p(gate), _p(logits), _p(shared), _p(slots), int(bool(mx8)))
    if rc < 0:
        raise ValueError("oracle_moe_layer: a selected expert has no blob")
    res = dict(out=out, idx=idx, gate=gate, order_dependent=rc)
    if want_stages:
        res.update(logits=logits, shared=shared, slots=slots)
    return res


def set_threads(n: int = 0) -> int:
    """Host threads for the layer's expert evaluations (0: leave as is);
    returns the number in effect.  Results do not depend on it."""
    return int(_load().oracle_set_threads(int(n)))


def to_bf16(a):
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_to_bf16(_p(a), a.size, _p(out))
    return out


def rmsnorm_bf16(h, eps=1e-6):
    h = _c(h, np.float32)
    B, H = h.reshape(-1, h.shape[-1]).shape
    out = np.empty((B, H), np.uint16)
    _load().oracle_rmsnorm_bf16(_p(h), B, H, float(eps), _p(out))
    return out


def dense_gemv_bf16(w, x):
    w = _c(w, np.uint16)
    N, K = w.shape
    x = _c(x, np.uint16).reshape(-1, K)
    y = np.empty((x.shape[0], N), np.uint16)
    _load().oracle_dense_gemv_bf16(_p(w), N, K, _p(x), x.shape[0], _p(y))
    return y
