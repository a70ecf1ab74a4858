"""The packed expert layout (moe_pack_experts / moe_unpack_experts).

A numpy model of the layout, written from the header's description, pins
the device rewrite byte for byte; the rewrite must be an exact, size-keeping
permutation of the canonical blob."""
import numpy as np
import pytest

import memory_bound_mxfp4_amd as moe
import synth


def canonical_parts(blob, H, I):
    """(codes, scales) of gate, up, down from a canonical blob."""
    off = synth.expert_offsets(H, I)
    g = blob[off[0]:off[0] + I * H // 2].reshape(I, H // 2)
    u = blob[off[1]:off[1] + I * H // 2].reshape(I, H // 2)
    d = blob[off[2]:off[2] + H * I // 2].reshape(H, I // 2)
    gs = blob[off[3]:off[3] + I * H // 32].reshape(I, H // 32)
    us = blob[off[4]:off[4] + I * H // 32].reshape(I, H // 32)
    ds = blob[off[5]:off[5] + H * I // 32].reshape(H, I // 32)
    return (g, gs), (u, us), (d, ds)


# In a full tile, byte 4 q + kb of a row's 16 scale bytes holds block 4 kb + q.
FULL_SCALE_ORDER = np.array([4 * (pos % 4) + pos // 4 for pos in range(16)])


def tile(codes, scales, g, s):
    """Packed tile (g, s) of one matrix: codes [SC][16 rows][16 B], then scales [16 rows][SC]
    (a full tile's row of 16 scale bytes in FULL_SCALE_ORDER)."""
    C = scales.shape[1]
    SC = min(16, C - 16 * s)
    rows = slice(16 * g, 16 * g + 16)
    cb = codes[rows].reshape(16, C, 16)[:, 16 * s:16 * s + SC, :]   # [row][block][16 B]
    sb = scales[rows, 16 * s:16 * s + SC]                             # [row][block]
    if SC == 16:
        sb = sb[:, FULL_SCALE_ORDER]
    return np.concatenate([cb.transpose(1, 0, 2).reshape(-1), sb.reshape(-1)])


def pack_ref(blob, H, I):
    (g, gs), (u, us), (d, ds) = canonical_parts(blob, H, I)
    parts = []
    C1, C2 = H // 32, I // 32
    for gi in range(I // 16):
        for s in range((C1 + 15) // 16):
            parts += [tile(g, gs, gi, s), tile(u, us, gi, s)]
    for gi in range(H // 16):
        for s in range((C2 + 15) // 16):
            parts.append(tile(d, ds, gi, s))
    body = np.concatenate(parts)
    out = np.zeros_like(blob)
    out[:body.size] = body
    return out


@pytest.mark.parametrize("H,I", [(256, 64), (96, 544), (1024, 512)])
def test_pack_ref_is_a_size_keeping_permutation(H, I):
    nb = synth.expert_bytes(H, I)
    blob = synth.expert_blob(5, 0, 3, H, I, 0.02)
    assert blob.size == nb
    packed = pack_ref(blob, H, I)
    assert packed.size == nb
    # every used byte lands somewhere exactly once: compare as multisets of
    # (value) and, stronger, pack a blob of distinct byte indices
    idx = np.arange(nb, dtype=np.int64)
    (g, gs), (u, us), (d, ds) = canonical_parts(idx, H, I)
    used = np.concatenate([x.reshape(-1) for x in (g, gs, u, us, d, ds)])
    p_idx = pack_ref(idx, H, I)[:used.size]
    assert np.array_equal(np.sort(p_idx), np.sort(used))


def test_pack_ref_first_tile_by_hand():
    """Tile (0, 0) of the gate matrix: block c of row r at c*256 + r*16."""
    H, I = 7168, 1536
    blob = synth.expert_blob(1, 0, 0, H, I, 0.02)
    (g, gs), _, _ = canonical_parts(blob, H, I)
    p = pack_ref(blob, H, I)
    for c, r in ((0, 0), (0, 15), (3, 7), (15, 2)):
        assert np.array_equal(p[c * 256 + r * 16:c * 256 + r * 16 + 16], g[r, 16 * c:16 * c + 16])
        assert p[4096 + r * 16 + 4 * (c % 4) + c // 4] == gs[r, c]  # block c = 4 kb + q at byte 4 q + kb
    # the up tile of (0, 0) follows the gate tile
    _, (u, us), _ = canonical_parts(blob, H, I)
    assert np.array_equal(p[4352:4352 + 16], u[0, :16])


@pytest.mark.gpu
@pytest.mark.parametrize("H,I,E", [(256, 64, 3), (7168, 1536, 2), (96, 544, 2)])
def test_device_pack_matches_reference_and_inverts(H, I, E):
    import torch
    print(f"[case] pack H={H} I={I} E={E}", flush=True)
    nb = synth.expert_bytes(H, I)
    host = np.concatenate([synth.expert_blob(9, 0, e, H, I, 0.02) for e in range(E)])
    dev = torch.from_numpy(host.copy()).cuda()
    moe.pack_experts(dev, E, H, I)
    got = dev.cpu().numpy()
    for e in range(E):
        assert np.array_equal(got[e * nb:(e + 1) * nb], pack_ref(host[e * nb:(e + 1) * nb], H, I)), e
    moe.unpack_experts(dev, E, H, I)
    assert np.array_equal(dev.cpu().numpy(), host)
