"""The entry point that allocates nothing (moe_decode_layer_noalloc): on the
library's static device workspace it gives exactly what moe_decode_layer
gives on a caller's workspace -- same indices, gates and residual, bit for
bit -- on two calls in a row, the second with a smaller batch, and it
rejects a batch whose workspace exceeds its array before launching."""
import numpy as np
import pytest

import memory_bound_mxfp4_amd as moe
from layer_inputs import residual_from_x, x_host
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(w, cfg, B, variant):
    import torch
    x = _dev(x_host(cfg, 0, variant=variant, batch=B))
    res0 = residual_from_x(x_host(cfg, 0, variant=variant, batch=B))
    r_ref = _dev(res0.copy())
    idx_ref, gate_ref = moe.moe_decode_layer(w, x, r_ref)
    r = _dev(res0.copy())
    idx = torch.full((B, w.top_k), -1, dtype=torch.int32, device="cuda")
    gate = torch.zeros((B, w.top_k), dtype=torch.float32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    moe.moe_decode_layer_noalloc(w, x, r, idx, gate, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(idx, idx_ref)
    assert torch.equal(gate.view(torch.int32), gate_ref.view(torch.int32))
    assert torch.equal(r.view(torch.int32), r_ref.view(torch.int32))
    return idx.cpu().numpy()


def test_noalloc_matches_workspace_entry_point(k3_layer):
    cfg = CONFIGS["k3_b8"]
    print("[case] no-alloc K3 B8 then B1 vs moe_decode_layer", flush=True)
    _both(k3_layer, cfg, 8, 21)
    _both(k3_layer, cfg, 1, 22)  # smaller batch on the array the batch-8 call left behind
    print("[case] no-alloc K3 B16 then B2", flush=True)
    _both(k3_layer, cfg, 16, 23)
    _both(k3_layer, cfg, 2, 24)


def test_noalloc_rejects_a_batch_beyond_its_array(k3_layer):
    import torch
    assert moe.workspace_size(k3_layer, 20) <= moe.NOALLOC_SCRATCH_BYTES < moe.workspace_size(k3_layer, 21)
    x = torch.zeros((21, k3_layer.hidden), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((21, k3_layer.hidden), dtype=torch.float32, device="cuda")
    idx = torch.zeros((21, k3_layer.top_k), dtype=torch.int32, device="cuda")
    gate = torch.zeros((21, k3_layer.top_k), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_layer_noalloc(k3_layer, x, r, idx, gate)
    assert e.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
