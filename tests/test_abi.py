"""The C ABI: the library loads without a GPU, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import memory_bound_mxfp4_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("router_topk", "expert_gemv_mxfp4", "moe_decode_layer", "moe_expert_bytes",
                     "moe_workspace_size", "moe_status_string"):
        assert required in names
    assert sorted(moe.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_expert_bytes_and_status_strings():
    assert moe.expert_bytes(7168, 1536) == 17547264 == oracle.expert_bytes(7168, 1536)
    assert moe.expert_bytes(256, 64) == 26112
    assert moe.expert_bytes(100, 64) == 0 and moe.expert_bytes(0, 32) == 0
    for s, name in ((0, "MOE_OK"), (-1, "MOE_ERR_INVALID_ARGUMENT"), (-2, "MOE_ERR_UNSUPPORTED"),
                    (-3, "MOE_ERR_WORKSPACE_TOO_SMALL"), (-4, "MOE_ERR_HIP")):
        assert moe.status_string(s) == name


class FakeTensor:
    """Stands in for a device tensor: only data_ptr() is used by the binding."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _weights(**over):
    base = dict(hidden=7168, inter=1536, num_experts=896, top_k=16, shared_inter=1536,
                router_w=FakeTensor(0x10000), experts=FakeTensor(0x20000), router_bias=None,
                shared_gate=FakeTensor(0x30000), shared_up=FakeTensor(0x40000), shared_down=FakeTensor(0x50000),
                expert_layout=moe.MOE_EXPERTS_PACKED)
    base.update(over)
    return moe.LayerWeights(**base)


def _ws_status(w, batch):
    n = ctypes.c_size_t(0)
    cs = w.c_struct()
    return moe.load().moe_workspace_size(ctypes.byref(cs), batch, ctypes.byref(n)), n.value


def test_workspace_size_and_argument_errors():
    st, n = _ws_status(_weights(), 1)
    assert st == moe.MOE_OK and n > 0
    st64, n64 = _ws_status(_weights(), 64)
    assert st64 == moe.MOE_OK and n64 > n
    bad = [
        (_weights(hidden=7000), 1),                 # H % 32
        (_weights(inter=1500), 1),                  # I % 32
        (_weights(), 0), (_weights(), 65),          # batch outside 1..64
        (_weights(top_k=897), 1),                   # k > E
        (_weights(top_k=0), 1),
        (_weights(router_w=FakeTensor(0)), 1),      # NULL
        (_weights(experts=FakeTensor(0x20010)), 1),  # blob base not 256-aligned
        (_weights(shared_down=FakeTensor(0)), 1),   # partial shared expert
        (_weights(shared_inter=0), 1),              # Is == 0 but pointers given
        (_weights(expert_layout=2), 1),             # unknown expert layout
    ]
    for w, b in bad:
        assert _ws_status(w, b)[0] == moe.MOE_ERR_INVALID_ARGUMENT, (w, b)
    assert _ws_status(_weights(hidden=32768), 1)[0] == moe.MOE_ERR_UNSUPPORTED
    assert _ws_status(_weights(shared_inter=0, shared_gate=None, shared_up=None, shared_down=None), 1)[0] == 0


def test_entry_points_reject_bad_arguments_before_launch():
    lib = moe.load()
    P = ctypes.c_void_p
    cs = _weights().c_struct()
    x, r, i, g, ws = P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x100000)
    # NULL x / residual / workspace
    assert lib.moe_decode_layer(ctypes.byref(cs), None, r, 1, i, g, ws, 1 << 30, None) == -1
    assert lib.moe_decode_layer(ctypes.byref(cs), x, None, 1, i, g, ws, 1 << 30, None) == -1
    assert lib.moe_decode_layer(ctypes.byref(cs), x, r, 1, i, g, None, 1 << 30, None) == -1
    # short workspace
    assert lib.moe_decode_layer(ctypes.byref(cs), x, r, 1, i, g, ws, 16, None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # misaligned workspace
    assert lib.moe_decode_layer(ctypes.byref(cs), x, r, 1, i, g, P(0x100010), 1 << 30, None) == -1
    # the layer streams packed experts only
    cs_canon = _weights(expert_layout=moe.MOE_EXPERTS_CANONICAL).c_struct()
    assert lib.moe_decode_layer(ctypes.byref(cs_canon), x, r, 1, i, g, ws, 1 << 30, None) == moe.MOE_ERR_UNSUPPORTED
    # pack/unpack: NULL, bad shapes, short or overlapping scratch
    nb = moe.expert_bytes(7168, 1536)
    assert lib.moe_pack_experts(None, 2, 7168, 1536, P(0x100000000), nb, None) == -1
    assert lib.moe_pack_experts(P(0x200000000), 2, 7000, 1536, P(0x100000000), nb, None) == -1
    assert lib.moe_unpack_experts(P(0x200000000), 0, 7168, 1536, P(0x100000000), nb, None) == -1
    assert lib.moe_pack_experts(P(0x200000000), 2, 7168, 1536, P(0x100000000), nb - 1, None) == -3
    assert lib.moe_pack_experts(P(0x200000000), 2, 7168, 1536, P(0x200000000 + nb), nb, None) == -1
    # router_topk: k > E, batch 0, H % 32
    assert lib.router_topk(x, 1, 7168, P(0x5000), None, 8, 9, i, g, P(0x6000), None, 0, None) == -1
    assert lib.router_topk(x, 0, 7168, P(0x5000), None, 896, 16, i, g, P(0x6000), None, 0, None) == -1
    assert lib.router_topk(x, 1, 7000, P(0x5000), None, 896, 16, i, g, P(0x6000), None, 0, None) == -1
    # router_topk without logits needs a workspace big enough for them
    assert lib.router_topk(x, 1, 7168, P(0x5000), None, 896, 16, i, g, None, ws, 64, None) == -3
    # expert_gemv_mxfp4: k % 32, bad dtype, batch 65
    assert lib.expert_gemv_mxfp4(P(0x1000), P(0x2000), 16, 48, x, 0, 1, P(0x3000), None) == -1
    assert lib.expert_gemv_mxfp4(P(0x1000), P(0x2000), 16, 64, x, 7, 1, P(0x3000), None) == -1
    assert lib.expert_gemv_mxfp4(P(0x1000), P(0x2000), 16, 64, x, 0, 65, P(0x3000), None) == -1
    # dense pieces
    assert lib.dense_gemv_bf16(P(0x1000), 16, 12, x, 1, P(0x3000), None) == -1
    assert lib.rmsnorm_bf16(None, 1, 16, ctypes.c_float(1e-6), P(0x3000), None) == -1
    assert lib.residual_add_bf16(P(0x1000), None, 1, 16, None) == -1
    # workspace status: NULL, misaligned, a buffer smaller than the control block
    assert lib.moe_workspace_status(None, 4096, P(0x3000), None) == -1
    assert lib.moe_workspace_status(ws, 4096, None, None) == -1
    assert lib.moe_workspace_status(P(0x100010), 4096, P(0x3000), None) == -1
    assert lib.moe_workspace_status(ws, 256, P(0x3000), None) == -1
    assert lib.moe_workspace_status(ws, 4096, P(0x3002), None) == -1
    # grid cap: negative counts are rejected; 0 (the default) is accepted
    assert lib.moe_set_max_workgroups(-1) == -1
    assert lib.moe_set_max_workgroups(0) == 0
    # stream-read probe: NULL, size not a multiple of 16, grid shape outside 1..32 blocks per CU
    assert lib.moe_stream_read_probe(None, 1 << 20, 4, P(0x3000), None) == -1
    assert lib.moe_stream_read_probe(P(0x1000), 1000, 4, P(0x3000), None) == -1
    assert lib.moe_stream_read_probe(P(0x1000), 1 << 20, 0, P(0x3000), None) == -1
    assert lib.moe_stream_read_probe(P(0x1000), 1 << 20, 33, P(0x3000), None) == -1
    assert lib.moe_stream_read_probe(P(0x1000), 1 << 20, 4, None, None) == -1
    # prefetch: no table, empty or oversized table, unaligned or ragged range, block count
    R = moe.RangeC
    ok = (R * 1)(R(0x1000, 4096))
    assert lib.moe_prefetch(None, 1, 64, None) == -1
    assert lib.moe_prefetch(ok, 0, 64, None) == -1
    assert lib.moe_prefetch((R * 9)(*[R(0x1000, 4096)] * 9), 9, 64, None) == -1
    assert lib.moe_prefetch((R * 1)(R(0x1008, 4096)), 1, 64, None) == -1
    assert lib.moe_prefetch((R * 1)(R(0x1000, 4100)), 1, 64, None) == -1
    assert lib.moe_prefetch((R * 1)(R(None, 4096)), 1, 64, None) == -1
    assert lib.moe_prefetch(ok, 1, 0, None) == -1
