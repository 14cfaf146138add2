"""GPU parity of the strided entry point: q, k, v read in place from fused
QKV buffers (both orders of the 3 and NH axes) and head-major buffers, and
out written into a padded buffer, against the CPU oracle on contiguous
copies of the same values.  Same bar as tests/test_parity.py."""
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


def layout_views(q, k, v, layout):
    """Copies of q, k, v placed in a buffer of the given layout, returned as
    (B,T,H,W,NH,HD) views (the values are bitwise those of q, k, v)."""
    B, T, H, W, NH, HD = q.shape
    if layout == "fused_3_nh":       # (B,T,H,W,3,NH,HD)
        buf = torch.stack([q, k, v], dim=4).contiguous()
        views = [buf[:, :, :, :, i] for i in range(3)]
    elif layout == "fused_nh_3":     # (B,T,H,W,NH,3,HD)
        buf = torch.stack([q, k, v], dim=5).contiguous()
        views = [buf[:, :, :, :, :, i] for i in range(3)]
    elif layout == "head_major":     # (B,NH,T,H,W,HD)
        views = [x.permute(0, 4, 1, 2, 3, 5).contiguous().permute(0, 2, 3, 4, 1, 5)
                 for x in (q, k, v)]
    else:
        raise ValueError(layout)
    for x, y in zip(views, (q, k, v)):
        assert not x.is_contiguous() and x.stride(-1) == 1
        assert torch.equal(x, y)
    return views


CASES = [((1, 9, 13, 21, 2, 64), (3, 7, 7)),
         ((1, 12, 18, 22, 2, 64), (11, 11, 11)),
         ((2, 7, 11, 19, 2, 32), (3, 5, 7)),
         ((1, 7, 11, 19, 2, 128), (3, 7, 7)),
         ((1, 16, 24, 7, 2, 64), (3, 5, 7))]


@pytest.mark.parametrize("layout", ["fused_3_nh", "fused_nh_3", "head_major"])
@pytest.mark.parametrize("shape,ks", CASES, ids=lambda x: str(x).replace(" ", ""))
def test_strided_inputs(layout, shape, ks):
    print("case layout=%s shape=%s window=%s" % (layout, shape, ks), flush=True)
    q, k, v = make_inputs(shape, 500 + shape[5], "cuda")
    qs, ks_, vs = layout_views(q, k, v, layout)
    out = na.fwd(qs, ks_, vs, ks)
    torch.cuda.synchronize()
    compare(out, oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks), "%s %s %s" % (layout, shape, ks))


# large-window instantiations, with their own grids: 4x4 blocks (5) and
# blocks of 2x4 queries on two planes (59, and 60 at head dim 128), whose
# q and out addresses add a plane step per lane
LARGE = {5: ((1, 12, 18, 22, 2, 64), (11, 11, 11)), 59: ((1, 12, 18, 22, 2, 64), (11, 11, 11)),
         60: ((1, 11, 20, 24, 1, 128), (11, 11, 11))}


@pytest.mark.parametrize("fam,var", [(1, 0), (2, 35), (2, 26), (2, 5), (2, 34), (2, 59), (2, 60)])
def test_strided_each_family(fam, var):
    """Fused-QKV inputs and a padded output through the general family and
    several rolling instantiations (border shifts, ragged tiles)."""
    shape, ks = LARGE.get(var, ((1, 9, 13, 21, 2, 64), (3, 7, 7)))
    print("case family=%d variant=%d shape=%s window=%s" % (fam, var, shape, ks), flush=True)
    q, k, v = make_inputs(shape, 600 + var, "cuda")
    qs, ks_, vs = layout_views(q, k, v, "fused_3_nh")
    pad = torch.full(shape[:5] + (shape[5] + 16,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = pad[..., :shape[5]]
    na.fwd(qs, ks_, vs, ks, out=out, config=(fam, var, 0))
    torch.cuda.synchronize()
    compare(out, oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks), "family %d variant %d" % (fam, var))
    assert bool((pad[..., shape[5]:] == 7.0).all()), "write outside the output view"


def test_strided_matches_contiguous_bitwise():
    """The same values through the contiguous and the strided entry points
    give bitwise equal outputs (same kernel, same summation order)."""
    shape, ks = (1, 16, 64, 96, 8, 64), (3, 7, 7)
    q, k, v = make_inputs(shape, 7, "cuda")
    a = na.fwd(q, k, v, ks)
    b = na.fwd(*layout_views(q, k, v, "fused_3_nh"), ks)
    c = na.fwd(*layout_views(q, k, v, "head_major"), ks)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_k_and_v_with_different_spatial_strides_are_rejected():
    shape, ks = (1, 6, 10, 12, 2, 64), (3, 5, 5)
    q, k, v = make_inputs(shape, 3, "cuda")
    qs, ks_, _ = layout_views(q, k, v, "fused_3_nh")
    with pytest.raises(na.NA3DError) as e:
        na.fwd(qs, ks_, v, ks)  # k fused, v contiguous
    assert e.value.status == na.NA3D_ERR_STRIDE
