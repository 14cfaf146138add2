"""Host-side contract and launch planning of the batched entry point
(na3d_fwd_batch): no GPU needed."""
import pytest

import neighborhood_attention_amd as na

MB = 1 << 20


def tiles_at(dims, NH=2, HD=64, base=0x10000000, gap=64 * MB):
    """Disjoint fake 16-B aligned addresses: q, k, v, out of tile i."""
    out = []
    for i, d in enumerate(dims):
        b = base + 4 * i * gap
        out.append((b, b + gap, b + 2 * gap, b + 3 * gap, d))
    return out


DIMS = [(1, 8, 32, 48), (1, 8, 32, 7), (2, 5, 16, 9)]


def check(tiles, NH=2, HD=64, ks=(3, 7, 7)):
    return na.check_args_batch(tiles, NH, HD, ks)


def test_valid_batches_pass():
    assert check(tiles_at(DIMS)) == na.NA3D_OK
    assert check([]) == na.NA3D_OK
    # tiles may share their inputs (only outputs must be disjoint)
    t = tiles_at(DIMS[:2])
    t[1] = (t[0][0], t[0][1], t[0][2], t[1][3], t[1][4])
    assert check(t) == na.NA3D_OK


def test_negative_count_and_null_array():
    lib = na.load()
    assert lib.na3d_check_args_batch(None, -1, 2, 64, 3, 7, 7) == na.NA3D_ERR_SHAPE
    assert lib.na3d_check_args_batch(None, 2, 2, 64, 3, 7, 7) == na.NA3D_ERR_NULL
    assert lib.na3d_check_args_batch(None, 0, 2, 64, 3, 7, 7) == na.NA3D_OK


@pytest.mark.parametrize("field", range(4))
def test_null_tensor_in_a_tile(field):
    t = tiles_at(DIMS)
    row = list(t[1])
    row[field] = 0
    t[1] = tuple(row)
    assert check(t) == na.NA3D_ERR_NULL


def test_window_must_fit_every_tile():
    assert check(tiles_at(DIMS + [(1, 8, 32, 5)])) == na.NA3D_ERR_WINDOW
    assert check(tiles_at([(1, 2, 32, 48)])) == na.NA3D_ERR_WINDOW


def test_head_dim_and_sizes():
    assert check(tiles_at(DIMS), HD=48) == na.NA3D_ERR_HEAD_DIM
    assert check(tiles_at([(0, 8, 32, 48)])) == na.NA3D_ERR_SHAPE


def test_alignment():
    t = tiles_at(DIMS)
    t[2] = (t[2][0] + 8,) + t[2][1:]
    assert check(t) == na.NA3D_ERR_ALIGN


def test_outputs_must_not_touch_other_tiles():
    t = tiles_at(DIMS)
    # out of tile 0 overlaps q of tile 1
    t0 = t[0]
    t[0] = (t0[0], t0[1], t0[2], t[1][0] + 4096, t0[4])
    assert check(t) == na.NA3D_ERR_OVERLAP
    # two tiles writing the same output
    t = tiles_at(DIMS)
    t[2] = t[2][:3] + (t[1][3], t[2][4])
    assert check(t) == na.NA3D_ERR_OVERLAP
    # out overlapping its own tile's input: same rule as na3d_fwd
    t = tiles_at(DIMS)
    t[0] = t[0][:3] + (t[0][2], t[0][4])
    assert check(t) == na.NA3D_ERR_OVERLAP


def test_plan_shares_one_launch():
    dims = [(1, 16, 64, 96)] * 2 + [(1, 16, 64, 7)] * 2 + [(1, 16, 32, 96), (1, 16, 32, 7)]
    p = na.plan_batch(dims, 8, 64, (3, 7, 7))
    assert p["launches"] == 1 and p["shared_tiles"] == 6
    assert p["variant"] == na.plan((1, 16, 64, 96, 8, 64), (3, 7, 7))["variant"]


def test_plan_splits_large_batches():
    p = na.plan_batch([(1, 8, 32, 48)] * 40, 2, 64, (3, 7, 7))
    assert p["launches"] == 3 and p["shared_tiles"] == 40


def test_plan_of_one_tile_matches_fwd():
    for shape, ks in (((1, 16, 64, 96, 8, 64), (3, 7, 7)), ((1, 16, 48, 64, 8, 64), (11, 11, 11)),
                      ((1, 32, 128, 192, 16, 128), (3, 7, 7))):
        p = na.plan_batch([shape[:4]], shape[4], shape[5], ks)
        single = na.plan(shape, ks)
        assert p["launches"] == 1
        assert p["variant"] == single["variant"]
        assert p["workgroups"] == single["workgroups"]


def test_plan_general_family_runs_tiles_alone():
    # a window whose halo no rolling instantiation's LDS holds at head dim
    # 128: every tile is its own launch
    p = na.plan_batch([(1, 24, 24, 24), (1, 20, 20, 20)], 2, 128, (19, 19, 19))
    assert na.plan((1, 24, 24, 24, 2, 128), (19, 19, 19))["family"] == 1
    assert p["launches"] == 2 and p["shared_tiles"] == 0 and p["variant"] == -1


def test_plan_empty():
    assert na.plan_batch([], 2, 64, (3, 7, 7)) == {"launches": 0, "variant": -1,
                                                   "shared_tiles": 0, "workgroups": 0}
