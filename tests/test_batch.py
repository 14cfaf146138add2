"""GPU parity of the batched entry point (na3d_fwd_batch, through the C
ABI): every tile of a batch against the CPU oracle on its own grid, and
bitwise against na3d_fwd run on that tile alone with the batch's rolling
instantiation (a query's arithmetic does not depend on how the grid is cut
into workgroups or launches)."""
import numpy as np
import pytest
import torch

import neighborhood_attention_amd as na
import oracle
from na3d_inputs import make_inputs

pytestmark = pytest.mark.gpu

REL_L2, MAX_ABS, REL_L2_EXPECTED = 1e-2, 5e-2, 4e-3


def compare(got, ref, what):
    got = got.detach().cpu().double().numpy()
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    mab = float(np.abs(diff).max())
    print("%s: rel_l2=%.3e max_abs=%.3e" % (what, rel, mab), flush=True)
    assert np.isfinite(got).all(), what
    assert rel <= REL_L2 and mab <= MAX_ABS and rel <= REL_L2_EXPECTED, (what, rel, mab)


def make_batch(dims, NH, HD, seed):
    return [make_inputs(tuple(d) + (NH, HD), seed + i, "cuda") for i, d in enumerate(dims)]


def check_batch(dims, NH, HD, ks, seed, oracle_check=True):
    print("case batch dims=%s NH=%d HD=%d window=%s seed=%d" % (dims, NH, HD, ks, seed), flush=True)
    qkv = make_batch(dims, NH, HD, seed)
    plan = na.plan_batch(dims, NH, HD, ks)
    outs = na.fwd_batch(qkv, ks)
    torch.cuda.synchronize()
    for i, ((q, k, v), o) in enumerate(zip(qkv, outs)):
        if oracle_check:
            compare(o, oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks), "tile %d %s" % (i, dims[i]))
        if plan["variant"] >= 0:
            alone = na.fwd(q, k, v, ks, config=(2, plan["variant"], 0))
        else:
            alone = na.fwd(q, k, v, ks)
        torch.cuda.synchronize()
        assert torch.equal(o, alone), ("tile", i, dims[i])
    return plan


def test_mixed_tile_sizes_one_launch():
    dims = [(1, 8, 32, 48), (1, 8, 32, 7), (2, 5, 16, 9), (1, 3, 7, 7), (1, 8, 7, 48)]
    plan = check_batch(dims, 2, 64, (3, 7, 7), 300)
    assert plan["launches"] == 1 and plan["shared_tiles"] == len(dims)


def test_decoder_like_mix_hd128():
    dims = [(1, 6, 24, 40), (1, 6, 24, 7), (1, 6, 9, 40)]
    plan = check_batch(dims, 2, 128, (3, 7, 7), 310)
    assert plan["launches"] == 1


def test_large_window_batch():
    dims = [(1, 12, 16, 20), (1, 11, 11, 11), (1, 12, 13, 24)]
    check_batch(dims, 1, 64, (11, 11, 11), 320)


@pytest.mark.parametrize("dims,HD,ks,shape_id", [
    # 12x4-query tiles of two-plane blocks (head dim 64, grids of 32+ planes)
    ([(1, 34, 20, 26), (1, 12, 13, 24), (1, 11, 11, 11)], 64, (11, 11, 11), (64, 8, 6, 2)),
    # 8x4-query tiles of two-plane blocks at head dim 128
    ([(1, 12, 16, 20), (1, 11, 11, 11)], 128, (11, 11, 11), (128, 8, 4, 2)),
    # 2x8 blocks in two 9-tile groups, eight phases along T, head dim 128
    ([(1, 14, 16, 24), (1, 13, 13, 13)], 128, (13, 13, 13), (128, 16, 1, 8)),
])
def test_multi_row_and_eight_phase_batches(dims, HD, ks, shape_id):
    plan = na.plan_batch(dims, 1, HD, ks)
    info = na.variant_info(plan["variant"])
    assert (info["hd"], info["qh"] * info["qw"], info["wh"], info["wt"]) == shape_id
    check_batch(dims, 1, HD, ks, 335)


def test_wide_window_batch():
    dims = [(1, 4, 8, 64), (1, 3, 5, 27)]
    check_batch(dims, 2, 64, (3, 5, 27), 330)


def test_more_tiles_than_one_launch_holds():
    dims = [(1, 3 + i % 4, 8 + i % 5, 8 + (7 * i) % 11) for i in range(21)]
    plan = check_batch(dims, 1, 32, (3, 5, 5), 340, oracle_check=False)
    assert plan["launches"] == 2 and plan["shared_tiles"] == 21


def test_general_family_batch():
    # no rolling instantiation holds this window's halo at head dim 128:
    # every tile runs alone
    dims = [(1, 22, 24, 24), (1, 20, 22, 23)]
    plan = check_batch(dims, 1, 128, (19, 19, 19), 350, oracle_check=False)
    assert plan["launches"] == 2 and plan["variant"] == -1


def test_four_group_window_batch():
    # the same window at head dim 64: one shared launch of the four-group
    # rolling instantiation
    dims = [(1, 22, 24, 24), (1, 20, 22, 23)]
    plan = check_batch(dims, 1, 64, (19, 19, 19), 355)
    assert plan["launches"] == 1 and plan["variant"] >= 0


def test_shared_inputs_and_given_outputs():
    q, k, v = make_inputs((1, 8, 16, 24, 2, 64), 360, "cuda")
    outs = [torch.full_like(q, 7.0) for _ in range(3)]
    res = na.fwd_batch([(q, k, v)] * 3, (3, 5, 5), outs=outs)
    torch.cuda.synchronize()
    assert all(r.data_ptr() == o.data_ptr() for r, o in zip(res, outs))
    alone = na.fwd(q, k, v, (3, 5, 5))
    for o in outs:
        assert torch.equal(o, alone)


def test_empty_and_errors():
    assert na.fwd_batch([], (3, 7, 7)) == []
    q, k, v = make_inputs((1, 4, 8, 8, 2, 64), 370, "cuda")
    q2, k2, v2 = make_inputs((1, 4, 8, 8, 4, 64), 371, "cuda")
    with pytest.raises(ValueError):
        na.fwd_batch([(q, k, v), (q2, k2, v2)], (3, 5, 5))    # NH differs
    with pytest.raises(na.NA3DError):
        na.fwd_batch([(q, k, v)], (5, 5, 5))                   # window exceeds T


def test_batch_is_repeatable():
    dims = [(1, 8, 32, 48), (1, 8, 32, 7)]
    qkv = make_batch(dims, 2, 64, 380)
    a = na.fwd_batch(qkv, (3, 7, 7))
    b = na.fwd_batch(qkv, (3, 7, 7))
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
