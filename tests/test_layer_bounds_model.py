"""Every address k_moe_layer computes stays inside its buffer, checked on the
CPU by a host model of the kernel's index arithmetic (layer_bounds_model.py)
for the routings that matter: all router rows equal (every logit of a row
tied, so every row picks experts 0..k-1 and, at batch 3, every active expert
has three rows), random routings, the ragged shapes (H and I not multiples of
512: clamped and masked tile loads) and batches that fill several column
groups of one expert."""
import numpy as np
import pytest

import layer_bounds_model as M
from layer_bounds_model import OutOfBounds, Shape, build_schedule, check_call, launch_shape


@pytest.mark.parametrize("k", [1, 3, 16, 33, 64])
@pytest.mark.parametrize("B", [1, 3])
def test_all_equal_router_rows(k, B):
    sh = Shape(H=256, I=64, E=896, k=k, Is=64, B=B)
    idx = [list(range(k)) for _ in range(B)]
    n = check_call(sh, idx)
    assert n > 0


@pytest.mark.parametrize("k", [1, 3, 16, 33, 64])
@pytest.mark.parametrize("B", [1, 3])
def test_random_routing(k, B):
    rng = np.random.default_rng(1000 * k + B)
    sh = Shape(H=256, I=64, E=896, k=k, Is=64, B=B)
    idx = [sorted(rng.choice(896, k, replace=False).tolist()) for _ in range(B)]
    check_call(sh, idx)


@pytest.mark.parametrize("B", [2, 17, 64])
def test_one_hot_expert_many_rows(B):
    """Every row routes to the same k experts (the last ones: highest blob
    offsets), so each active expert spreads over ceil(B/16) column groups."""
    k = 4
    sh = Shape(H=256, I=96, E=64, k=k, Is=32, B=B)
    idx = [list(range(64 - k, 64)) for _ in range(B)]
    check_call(sh, idx)


def test_ragged_shape_and_wide_column_groups():
    sh = Shape(H=544, I=96, E=40, k=5, Is=24, B=40)
    rng = np.random.default_rng(3)
    idx = [sorted(rng.choice(40, 5, replace=False).tolist()) for _ in range(40)]
    check_call(sh, idx)


def test_schedule_model_inverts_the_routing():
    sh = Shape(H=256, I=64, E=896, k=16, Is=64, B=3)
    idx = [list(range(16)) for _ in range(3)]
    s = build_schedule(sh, idx)
    assert s.U == 16 and s.active == list(range(16))
    assert s.row_off == list(range(0, 49, 3)) and s.cg_off == list(range(17))
    for a in range(16):
        assert sorted(s.rows[s.row_off[a]:s.row_off[a + 1]]) == [a, 16 + a, 32 + a]


def test_model_catches_an_access_past_a_buffer(monkeypatch):
    """The checker itself: a tile offset formula one tile too far is caught."""
    import layer_bounds_model as m
    sh = Shape(H=256, I=64, E=16, k=2, Is=64, B=1)
    orig = m.tile_off
    monkeypatch.setattr(m, "tile_off", lambda g, s, C: orig(g, s, C) + 16 * C * 17 * 64)
    with pytest.raises(OutOfBounds):
        check_call(sh, [[14, 15]])


def test_lds_layout_matches_the_kernel_constants():
    ls = launch_shape(Shape(H=7168, I=1536, E=896, k=16, Is=1536, B=1))
    assert ls["full"] and ls["rg"] == 1
    ls64 = launch_shape(Shape(H=7168, I=1536, E=896, k=16, Is=1536, B=64))
    assert ls64["full"] and ls64["rg"] == 4 and ls64["lds_h_off"] >= 33280


def test_batch1_fc1_segments_cover_each_segment_once():
    """The batch-1 routed FC1 segment map gives every segment of a row group to
    exactly one (wave, pass); at H 7168 (14 segments) the waves take 4, 4, 3
    and 3 passes, and the two with an even count hand their buffers on."""
    for S1 in range(1, 80):
        seen = []
        for w in range(4):
            seen += [M.fc1_seg(w, p) for p in range(M.fc1_passes(S1, w))]
        assert sorted(seen) == list(range(S1))
    assert [M.fc1_passes(14, w) for w in range(4)] == [4, 4, 3, 3]
