"""Host-only checks of the query-box entry point (no GPU needed)."""
import pytest

import neighborhood_attention_amd as na

GRID = (2, 6, 10, 12, 2, 32)   # k and v: (B, T, H, W, NH, HD)
KS = (3, 5, 5)
BASE = 0x100000


def nbytes(shape):
    n = 2
    for x in shape:
        n *= x
    return n


def ptrs_for(box):
    qshape = GRID[:1] + tuple(box[3:]) + GRID[4:]
    nq, nk = nbytes(qshape), nbytes(GRID)
    return (BASE, BASE + nq, BASE + nq + nk, BASE + nq + 2 * nk)


@pytest.mark.parametrize("box", [(0, 0, 0, 6, 10, 12), (1, 2, 3, 4, 5, 6), (5, 9, 11, 1, 1, 1),
                                 (0, 0, 7, 6, 10, 5)])
def test_boxes_inside_the_grid_pass(box):
    assert na.check_args_subgrid(*ptrs_for(box), GRID, KS, box) == na.NA3D_OK


@pytest.mark.parametrize("box", [(0, 0, 0, 7, 10, 12), (0, 0, 0, 6, 11, 12), (0, 0, 0, 6, 10, 13),
                                 (-1, 0, 0, 2, 2, 2), (0, -1, 0, 2, 2, 2), (0, 0, -1, 2, 2, 2),
                                 (5, 0, 0, 2, 2, 2), (0, 9, 0, 1, 2, 1), (0, 0, 12, 1, 1, 1),
                                 (0, 0, 0, 0, 2, 2), (0, 0, 0, 2, 0, 2), (0, 0, 0, 2, 2, 0)])
def test_boxes_outside_the_grid_are_rejected(box):
    ptrs = ptrs_for((0, 0, 0, 1, 1, 1))
    assert na.check_args_subgrid(*ptrs, GRID, KS, box) == na.NA3D_ERR_BOX


def test_null_box():
    lib = na.load()
    assert lib.na3d_check_args_subgrid(*ptrs_for((0, 0, 0, 1, 1, 1)), *GRID, *KS, None,
                                       None) == na.NA3D_ERR_NULL


def test_window_and_head_dim_checks_still_apply():
    box = (0, 0, 0, 2, 2, 2)
    assert na.check_args_subgrid(*ptrs_for(box), GRID, (7, 5, 5), box) == na.NA3D_ERR_WINDOW
    assert na.check_args_subgrid(*ptrs_for(box), GRID[:5] + (48,), KS, box) == na.NA3D_ERR_HEAD_DIM


def test_output_overlap_uses_the_box_extent():
    box = (1, 2, 3, 2, 3, 4)
    q, k, v = BASE, BASE + (1 << 24), BASE + (2 << 24)
    qshape = GRID[:1] + box[3:] + GRID[4:]
    # out right after q's (box-sized) span: fine; one row earlier: overlap
    assert na.check_args_subgrid(q, k, v, q + nbytes(qshape), GRID, KS, box) == na.NA3D_OK
    assert na.check_args_subgrid(q, k, v, q + nbytes(qshape) - 64, GRID, KS, box) == \
        na.NA3D_ERR_OVERLAP


def test_box_views_of_the_full_query_tensor():
    """q as a strided view of a whole-grid q tensor (offset base, grid strides)."""
    B, T, H, W, NH, HD = GRID
    box = (1, 2, 3, 2, 3, 4)
    sn, sw = HD, NH * HD
    sh, st, sb = W * sw, H * W * sw, T * H * W * sw
    grid_st = (sb, st, sh, sw, sn)
    nk = nbytes(GRID)
    qbase = BASE + 2 * (box[0] * st + box[1] * sh + box[2] * sw)
    out = BASE + 3 * nk
    ob = (B, box[3], box[4], box[5], NH, HD)
    ost = (box[3] * box[4] * box[5] * NH * HD, box[4] * box[5] * NH * HD, box[5] * NH * HD,
           NH * HD, HD)
    assert na.check_args_subgrid(qbase, BASE + nk, BASE + 2 * nk, out, GRID, KS, box,
                                 [grid_st, grid_st, grid_st, ost]) == na.NA3D_OK
    assert nbytes(ob) < nk
