"""GPU parity of the query-box entry point: queries of a sub-box of the grid,
windows placed in the whole grid, against the CPU oracle on the whole grid
restricted to the box.  Same bar as tests/test_parity.py."""
import numpy as np
import pytest
import torch

import neighborhood_attention_amd as na
import oracle
from na3d_inputs import make_inputs

pytestmark = pytest.mark.gpu

REL_L2, MAX_ABS, REL_L2_EXPECTED = 1e-2, 5e-2, 4e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    na.load()


def compare(got, ref, what):
    got = got.detach().to("cpu").to(torch.float64).numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), what
    diff = got - ref
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    mab = float(np.abs(diff).max())
    print("%s: rel_l2=%.3e max_abs=%.3e" % (what, rel, mab), flush=True)
    assert rel <= REL_L2 and mab <= MAX_ABS and rel <= REL_L2_EXPECTED, (what, rel, mab)


def sl(box):
    t0, h0, w0, tq, hq, wq = box
    return (slice(None), slice(t0, t0 + tq), slice(h0, h0 + hq), slice(w0, w0 + wq))


GRIDS = [((1, 9, 13, 21, 2, 64), (3, 7, 7)),
         ((1, 12, 18, 22, 2, 64), (11, 11, 11)),
         ((2, 7, 11, 19, 2, 32), (3, 5, 7)),
         ((1, 7, 11, 19, 2, 128), (3, 7, 7))]

BOXES = ["full", "interior", "corner", "w_tail", "thin_t", "one_query"]


def make_box(name, shape, ks):
    B, T, H, W, NH, HD = shape
    return {
        "full": (0, 0, 0, T, H, W),
        "interior": (1, 2, 3, T - 2, H - 4, W - 5),
        "corner": (T - 3, H - 5, W - 6, 3, 5, 6),
        "w_tail": (0, 0, W - 5, T, H, 5),          # the pages' W sub-slice case
        "thin_t": (T // 2, 1, 0, 1, H - 2, W),
        "one_query": (T - 1, 0, W // 2, 1, 1, 1),
    }[name]


@pytest.mark.parametrize("box_name", BOXES)
@pytest.mark.parametrize("shape,ks", GRIDS, ids=lambda x: str(x).replace(" ", ""))
def test_subgrid(box_name, shape, ks):
    box = make_box(box_name, shape, ks)
    print("case box=%s %s shape=%s window=%s" % (box_name, box, shape, ks), flush=True)
    q, k, v = make_inputs(shape, 700 + shape[5], "cuda")
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks)[sl(box)]
    qb = q[sl(box)]                            # strided view into the whole q
    out = na.fwd_subgrid(qb, k, v, ks, box[:3])
    out2 = na.fwd_subgrid(qb.contiguous(), k, v, ks, box[:3])
    torch.cuda.synchronize()
    compare(out, ref, "box %s %s" % (box_name, box))
    assert torch.equal(out, out2)


# large-window instantiations, with their own grids: 4x4 blocks (5) and
# blocks of 2x4 queries on two planes (59, and 60 at head dim 128; the box
# has an odd number of planes, so a block's second plane can lie past it)
LARGE = {5: ((1, 12, 18, 22, 2, 64), (11, 11, 11)), 59: ((1, 12, 18, 22, 2, 64), (11, 11, 11)),
         60: ((1, 12, 20, 24, 1, 128), (11, 11, 11))}


@pytest.mark.parametrize("fam,var", [(1, 0), (2, 35), (2, 26), (2, 5), (2, 34), (2, 21), (2, 59),
                                     (2, 60)])
def test_subgrid_each_family(fam, var):
    shape, ks = LARGE.get(var, ((1, 9, 13, 21, 2, 64), (3, 7, 7)))
    box = (2, 3, 5, shape[1] - 3, shape[2] - 5, shape[3] - 9)
    print("case family=%d variant=%d box=%s" % (fam, var, box), flush=True)
    q, k, v = make_inputs(shape, 800 + var, "cuda")
    out = na.fwd_subgrid(q[sl(box)], k, v, ks, box[:3], config=(fam, var, 0))
    torch.cuda.synchronize()
    compare(out, oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks)[sl(box)],
            "family %d variant %d" % (fam, var))


def test_split_grid_reassembles_the_whole():
    """The decoder tile's queries split into 2 x 2 boxes along H and W (the
    per-GPU share of a spatial split) reassemble the whole-grid result."""
    shape, ks = (1, 16, 64, 96, 8, 64), (3, 7, 7)
    q, k, v = make_inputs(shape, 11, "cuda")
    whole = na.fwd(q, k, v, ks)
    parts = torch.empty_like(whole)
    for h0 in (0, 32):
        for w0 in (0, 48):
            box = (0, h0, w0, 16, 32, 48)
            na.fwd_subgrid(q[sl(box)], k, v, ks, box[:3], out=parts[sl(box)])
    torch.cuda.synchronize()
    a = whole.to(torch.float64)
    d = (parts.to(torch.float64) - a)
    rel = float(d.norm() / a.norm())
    print("split vs whole: rel %.3e max %.3e" % (rel, float(d.abs().max())), flush=True)
    assert rel < 2e-3 and float(d.abs().max()) < 2e-2


def test_box_outside_grid_raises():
    shape, ks = (1, 6, 10, 12, 2, 64), (3, 5, 5)
    q, k, v = make_inputs(shape, 3, "cuda")
    with pytest.raises(na.NA3DError) as e:
        na.fwd_subgrid(q[:, :3, :4, :5], k, v, ks, (4, 0, 0))   # t0 + Tq > T
    assert e.value.status == na.NA3D_ERR_BOX
