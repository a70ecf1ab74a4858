"""Python binding of libmoe_mxfp4.so, the MI355X MXFP4 MoE decode-layer library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (bf16 data may be
torch.bfloat16 or int16/uint16 bit patterns); work goes on the current torch
stream unless a stream is given.  If the library is not built, loading
raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mxfp4.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_DTYPE_BF16, MOE_DTYPE_F32 = 0, 1
MOE_EXPERTS_CANONICAL, MOE_EXPERTS_PACKED = 0, 1
MAX_BATCH = 64

# Symbols the C header declares (checked by tests/test_abi.py).
EXPORTS = ("moe_expert_bytes", "moe_workspace_size", "moe_router_workspace_size", "router_topk",
           "expert_gemv_mxfp4", "moe_decode_layer", "moe_decode_layer_kernel_count",
           "moe_decode_layer_kernel_name", "moe_decode_layer_timed", "moe_workspace_init", "moe_pack_experts",
           "moe_unpack_experts", "rmsnorm_bf16", "dense_gemv_bf16", "residual_add_bf16", "residual_add_rmsnorm_bf16",
           "moe_workspace_status", "moe_stream_read_probe", "moe_decode_layer_noalloc", "moe_decode_layer_mxfp8",
           "moe_prefetch", "moe_set_max_workgroups", "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class LayerWeightsC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("shared_gate", ctypes.c_void_p), ("shared_up", ctypes.c_void_p),
                ("shared_down", ctypes.c_void_p), ("experts", ctypes.c_void_p), ("expert_layout", ctypes.c_int32)]


_lib = None


def load():
    """Load the built library (raises if it is missing: no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run memory_bound_mxfp4_amd.build.build() "
                          "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    sig = {
        "moe_expert_bytes": (Z, [I, I]),
        "moe_workspace_size": (I, [P, I, ctypes.POINTER(Z)]),
        "moe_router_workspace_size": (Z, [I, I]),
        "router_topk": (I, [P, I, I, P, P, I, I, P, P, P, P, Z, P]),
        "expert_gemv_mxfp4": (I, [P, P, I, I, P, I, I, P, P]),
        "moe_decode_layer": (I, [P, P, P, I, P, P, P, Z, P]),
        "moe_decode_layer_kernel_count": (I, []),
        "moe_decode_layer_kernel_name": (ctypes.c_char_p, [I]),
        "moe_decode_layer_timed": (I, [P, P, P, I, P, P, P, Z, P, P, I]),
        "moe_workspace_init": (I, [P, Z, P]),
        "moe_pack_experts": (I, [P, I, I, I, P, Z, P]),
        "moe_unpack_experts": (I, [P, I, I, I, P, Z, P]),
        "rmsnorm_bf16": (I, [P, I, I, F, P, P]),
        "dense_gemv_bf16": (I, [P, I, I, P, I, P, P]),
        "residual_add_bf16": (I, [P, P, I, I, P]),
        "residual_add_rmsnorm_bf16": (I, [P, P, I, I, F, P, P]),
        "moe_workspace_status": (I, [P, Z, P, P]),
        "moe_decode_layer_noalloc": (I, [P, P, P, I, P, P, P, P]),
        "moe_decode_layer_mxfp8": (I, [P, P, P, I, P, P, P, Z, P]),
        "moe_prefetch": (I, [P, I, I, P]),
        "moe_set_max_workgroups": (I, [I]),
        "moe_stream_read_probe": (I, [P, Z, I, P, P]),
        "moe_status_string": (ctypes.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def expert_bytes(hidden: int, inter: int) -> int:
    return int(load().moe_expert_bytes(hidden, inter))


@dataclass
class LayerWeights:
    """One layer's weights (device tensors) and shape."""
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    shared_inter: int
    router_w: object
    experts: object
    router_bias: Optional[object] = None
    shared_gate: Optional[object] = None
    shared_up: Optional[object] = None
    shared_down: Optional[object] = None
    expert_layout: int = MOE_EXPERTS_CANONICAL

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        if name != "_cs":
            object.__setattr__(self, "_cs", None)

    def c_struct(self) -> LayerWeightsC:
        cs = getattr(self, "_cs", None)
        if cs is not None:
            return cs
        cs = LayerWeightsC(self.hidden, self.inter, self.num_experts, self.top_k, self.shared_inter,
                             _ptr(self.router_w), _ptr(self.router_bias), _ptr(self.shared_gate),
                             _ptr(self.shared_up), _ptr(self.shared_down), _ptr(self.experts), self.expert_layout)
        object.__setattr__(self, "_cs", cs)
        return cs


def _pack(experts, num_experts: int, hidden: int, inter: int, to_packed: bool, scratch=None, stream=None):
    import torch
    nb = expert_bytes(hidden, inter)
    scratch = torch.empty(nb, dtype=torch.uint8, device=experts.device) if scratch is None else scratch
    f = load().moe_pack_experts if to_packed else load().moe_unpack_experts
    _check(f(_ptr(experts), num_experts, hidden, inter, _ptr(scratch), scratch.numel(), _stream(stream)),
           "moe_pack_experts" if to_packed else "moe_unpack_experts")
    return experts


def pack_experts(experts, num_experts: int, hidden: int, inter: int, scratch=None, stream=None):
    """Rewrite canonical expert blobs in place into the packed layout (moe_pack_experts)."""
    return _pack(experts, num_experts, hidden, inter, True, scratch, stream)


def unpack_experts(experts, num_experts: int, hidden: int, inter: int, scratch=None, stream=None):
    """Inverse of pack_experts (moe_unpack_experts)."""
    return _pack(experts, num_experts, hidden, inter, False, scratch, stream)


def pack_layer(w: LayerWeights, stream=None) -> LayerWeights:
    """Pack a layer's experts in place (once, at load time) and mark them packed."""
    if w.expert_layout != MOE_EXPERTS_PACKED:
        pack_experts(w.experts, w.num_experts, w.hidden, w.inter, stream=stream)
        w.expert_layout = MOE_EXPERTS_PACKED
    return w


def workspace_size(w: LayerWeights, batch: int) -> int:
    n = ctypes.c_size_t(0)
    cs = w.c_struct()
    _check(load().moe_workspace_size(ctypes.byref(cs), batch, ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


WS_STATUS_OFFSET = 28


def workspace_init(ws, stream=None):
    """Clear a workspace before its first use (moe_workspace_init)."""
    _check(load().moe_workspace_init(_ptr(ws), ws.numel(), _stream(stream)), "moe_workspace_init")
    return ws


def alloc_workspace(w: LayerWeights, batch: int, device=None):
    """A cleared workspace for `w` at `batch` rows."""
    import torch
    ws = torch.empty(workspace_size(w, batch), dtype=torch.uint8, device=device or w.router_w.device)
    return workspace_init(ws)


WS_ACTIVE_EXPERTS_OFFSET = 384


def workspace_status(ws, stream=None) -> int:
    """The workspace's sticky status word (0 = every wait completed), read
    through moe_workspace_status. Synchronises the stream."""
    import torch
    out = torch.zeros(1, dtype=torch.int32, device=ws.device)
    _check(load().moe_workspace_status(_ptr(ws), ws.numel(), _ptr(out), _stream(stream)), "moe_workspace_status")
    torch.cuda.synchronize(ws.device)
    return int(out.item()) & 0xFFFFFFFF


def workspace_active_experts(ws) -> int:
    """Batch > 1: distinct experts the last call on `ws` routed to, as counted
    on the device (low half of the word at WS_ACTIVE_EXPERTS_OFFSET). Synchronises."""
    import numpy as np
    off = WS_ACTIVE_EXPERTS_OFFSET
    return int(ws[off:off + 4].cpu().numpy().view(np.uint32)[0])


def set_max_workgroups(n: int) -> None:
    """Cap the layer kernel's grid at n workgroups (0: the default) -- moe_set_max_workgroups."""
    _check(load().moe_set_max_workgroups(int(n)), "moe_set_max_workgroups")


def stream_read_probe(buf, blocks_per_cu: int = 4, sink=None, stream=None):
    """Enqueue one streaming read of all of `buf` (moe_stream_read_probe)."""
    import torch
    sink = torch.zeros(1, dtype=torch.int32, device=buf.device) if sink is None else sink
    _check(load().moe_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), blocks_per_cu, _ptr(sink),
                                        _stream(stream)), "moe_stream_read_probe")
    return sink


def router_topk(x, router_w, top_k: int, bias=None, idx=None, gate=None, logits=None, ws=None, stream=None):
    """Router GEMV + top-k + renormalised gates. Returns (idx int32 [B][k], gate fp32 [B][k])."""
    import torch
    B, H = x.shape
    E = router_w.shape[0]
    dev = x.device
    idx = torch.empty((B, top_k), dtype=torch.int32, device=dev) if idx is None else idx
    gate = torch.empty((B, top_k), dtype=torch.float32, device=dev) if gate is None else gate
    if logits is None and ws is None:
        ws = torch.empty(load().moe_router_workspace_size(B, E), dtype=torch.uint8, device=dev)
    _check(load().router_topk(_ptr(x), B, H, _ptr(router_w), _ptr(bias), E, top_k, _ptr(idx), _ptr(gate),
                              _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "router_topk")
    return idx, gate


def expert_gemv_mxfp4(codes, scales, x, n: int, k: int, y=None, stream=None):
    """y[b][n] = dequant(codes, scales) . x[b]; x bf16 or fp32 [B][k]. Returns y fp32 [B][n]."""
    import torch
    B = x.shape[0]
    y = torch.empty((B, n), dtype=torch.float32, device=x.device) if y is None else y
    xdt = MOE_DTYPE_F32 if x.dtype == torch.float32 else MOE_DTYPE_BF16
    _check(load().expert_gemv_mxfp4(_ptr(codes), _ptr(scales), n, k, _ptr(x), xdt, B, _ptr(y), _stream(stream)),
           "expert_gemv_mxfp4")
    return y


def moe_decode_layer(w: LayerWeights, x, residual, idx=None, gate=None, ws=None, stream=None, mxfp8=False):
    """The whole layer; `residual` (fp32 [B][H]) is updated in place. Returns (idx, gate).
    mxfp8: the routed experts' FP4 x MXFP8 variant (moe_decode_layer_mxfp8)."""
    import torch
    B = x.shape[0]
    dev = x.device
    idx = torch.empty((B, w.top_k), dtype=torch.int32, device=dev) if idx is None else idx
    gate = torch.empty((B, w.top_k), dtype=torch.float32, device=dev) if gate is None else gate
    ws = alloc_workspace(w, B, dev) if ws is None else ws
    cs = w.c_struct()
    f, name = (load().moe_decode_layer_mxfp8, "moe_decode_layer_mxfp8") if mxfp8 else \
        (load().moe_decode_layer, "moe_decode_layer")
    _check(f(ctypes.byref(cs), _ptr(x), _ptr(residual), B, _ptr(idx), _ptr(gate), _ptr(ws), ws.numel(),
             _stream(stream)), name)
    return idx, gate


NOALLOC_SCRATCH_BYTES = 24 << 20


def moe_decode_layer_noalloc(w: LayerWeights, x, residual, idx, gate, status=None, stream=None):
    """moe_decode_layer on the library's own static device workspace
    (moe_decode_layer_noalloc): nothing is allocated by the call.  idx, gate
    and the optional status word (int32 [1]) are caller-provided device tensors."""
    B = x.shape[0]
    cs = w.c_struct()
    _check(load().moe_decode_layer_noalloc(ctypes.byref(cs), _ptr(x), _ptr(residual), B, _ptr(idx), _ptr(gate),
                                           _ptr(status), _stream(stream)), "moe_decode_layer_noalloc")
    return idx, gate


def layer_kernel_names():
    lib = load()
    return [lib.moe_decode_layer_kernel_name(i).decode() for i in range(lib.moe_decode_layer_kernel_count())]


def moe_decode_layer_timed(w: LayerWeights, x, residual, idx, gate, ws, events, stream=None):
    """moe_decode_layer recording torch.cuda.Event objects around each kernel
    (len(events) == len(layer_kernel_names()) + 1) on `stream`."""
    B = x.shape[0]
    cs = w.c_struct()
    for e in events:  # torch creates the underlying hipEvent_t lazily, on first record
        if not e.cuda_event:
            e.record()
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(load().moe_decode_layer_timed(ctypes.byref(cs), _ptr(x), _ptr(residual), B, _ptr(idx), _ptr(gate),
                                         _ptr(ws), ws.numel(), _stream(stream), arr, len(events)),
           "moe_decode_layer_timed")
    return idx, gate


class RangeC(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


PREFETCH_MAX_RANGES = 8


def prefetch(tensors, blocks: int = 256, stream=None):
    """Read device tensors once into the last-level cache (moe_prefetch)."""
    tensors = [t for t in tensors if t is not None]
    arr = (RangeC * len(tensors))(*[RangeC(t.data_ptr(), t.numel() * t.element_size()) for t in tensors])
    _check(load().moe_prefetch(arr, len(tensors), blocks, _stream(stream)), "moe_prefetch")


def rmsnorm_bf16(h, eps: float = 1e-6, out=None, stream=None):
    import torch
    B, H = h.shape
    out = torch.empty((B, H), dtype=torch.bfloat16, device=h.device) if out is None else out
    _check(load().rmsnorm_bf16(_ptr(h), B, H, float(eps), _ptr(out), _stream(stream)), "rmsnorm_bf16")
    return out


def dense_gemv_bf16(w, x, y=None, stream=None):
    import torch
    n, k = w.shape
    B = x.shape[0]
    y = torch.empty((B, n), dtype=torch.bfloat16, device=x.device) if y is None else y
    _check(load().dense_gemv_bf16(_ptr(w), n, k, _ptr(x), B, _ptr(y), _stream(stream)), "dense_gemv_bf16")
    return y


def residual_add_bf16(h, t, stream=None):
    B, H = h.shape
    _check(load().residual_add_bf16(_ptr(h), _ptr(t), B, H, _stream(stream)), "residual_add_bf16")
    return h


def residual_add_rmsnorm_bf16(h, t, eps: float = 1e-6, out=None, stream=None):
    """h += t (in place), then out = bf16(RMSNorm(h)), as one launch."""
    import torch
    B, H = h.shape
    out = torch.empty((B, H), dtype=torch.bfloat16, device=h.device) if out is None else out
    _check(load().residual_add_rmsnorm_bf16(_ptr(h), _ptr(t), B, H, float(eps), _ptr(out), _stream(stream)),
           "residual_add_rmsnorm_bf16")
    return out
