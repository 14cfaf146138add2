"""GPU parity of the bf16 RMSNorm kernel (through the C ABI) against the
fp64 oracle in oracle/rmsnorm.py, on the same seeded bf16 inputs.

Bound, element by element: the kernel's fp32 result is within a few fp32
roundings (< 2^-17 relative) of the exact value, and rounding it once to
bf16 adds at most 2^-8 relative, so |y - exact| <= (2^-8 + 2^-14) |exact|.
The whole-tensor tolerance of the attention path (rel-L2 <= 1e-2, max-abs
<= 5e-2) is checked as well."""
import numpy as np
import pytest

from oracle.rmsnorm import rms_norm as oracle_rms_norm

pytestmark = pytest.mark.gpu

ELEM_REL = 2.0 ** -8 + 2.0 ** -14


def _torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch


def _compare(y, x, w, eps, where):
    ref = oracle_rms_norm(x.float().cpu().numpy(), None if w is None else w.float().cpu().numpy(),
                          eps)
    got = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = ELEM_REL * np.abs(ref) + 1e-30
    bad = err > bound
    assert not bad.any(), "%s: %d elements beyond the bound, first at %s: got %r ref %r" % (
        where, int(bad.sum()), np.argwhere(bad)[0], got[bad][0], ref[bad][0])
    nref = np.linalg.norm(ref)
    if nref > 0:
        assert np.linalg.norm(got - ref) / nref <= 1e-2
    assert err.max(initial=0.0) <= 5e-2 * max(1.0, np.abs(ref).max(initial=0.0))
    return ref


CASES = [
    # rows, dim, weight, eps, workgroups
    (1, 8, True, 1e-6, None),        # smallest row: one piece, 63 idle lanes
    (5, 512, False, 1e-6, None),     # one piece per lane, no idle lane
    (37, 520, True, 1e-5, None),     # 65 pieces: second piece on lane 0 only
    (300, 1024, False, 1e-6, None),
    (129, 2056, True, 1e-6, None),   # 257 pieces: four per lane plus one
    (64, 4096, True, 1e-6, None),
    (1000, 3072, True, 0.5, None),   # 384 pieces, large eps
    (33, 8192, True, 1e-6, None),    # the largest row
    (17, 8184, False, 1e-6, None),
    (1000, 4096, True, 1e-6, 1),     # 4 waves walk all rows: both row buffers, odd tail
    (1001, 2048, True, 1e-6, 3),
    (999, 520, False, 1e-6, 7),
    (250, 4096, True, 1e-6, 10000),  # more waves than rows
]


@pytest.mark.parametrize("rows,dim,weighted,eps,wgs", CASES)
def test_parity(rows, dim, weighted, eps, wgs):
    torch = _torch()
    import neighborhood_attention_amd as na
    from na3d_inputs import make_norm_inputs

    x, w = make_norm_inputs(rows, dim, 100 + rows + dim, "cpu")
    xd, wd = x.cuda(), (w.cuda() if weighted else None)
    y = na.rms_norm(xd, wd, eps, workgroups=wgs)
    torch.cuda.synchronize()
    _compare(y, x, w if weighted else None, eps, "rows=%d dim=%d" % (rows, dim))


def test_grid_does_not_change_bits():
    torch = _torch()
    import neighborhood_attention_amd as na
    from na3d_inputs import make_norm_inputs

    x, w = make_norm_inputs(777, 4096, 7, "cuda")
    base = na.rms_norm(x, w)
    for g in (1, 2, 5, 64, 195, 4096):
        assert torch.equal(na.rms_norm(x, w, workgroups=g), base), g
    assert torch.equal(na.rms_norm(x, w), base)   # repeatable


def test_in_place():
    torch = _torch()
    import neighborhood_attention_amd as na
    from na3d_inputs import make_norm_inputs

    x, w = make_norm_inputs(513, 2048, 8, "cuda")
    expect = na.rms_norm(x, w)
    for g in (None, 1, 3):
        xi = x.clone()
        out = na.rms_norm(xi, w, out=xi, workgroups=g)
        torch.cuda.synchronize()
        assert out.data_ptr() == xi.data_ptr()
        assert torch.equal(xi, expect), g


def test_special_rows():
    """Rows with closed-form results, through the kernel."""
    torch = _torch()
    import neighborhood_attention_amd as na

    dim = 1536
    x = torch.zeros((6, dim), dtype=torch.float32)
    x[1] = 3.0                                     # constant row
    x[2, 100] = -2.5                               # one non-zero element
    x[3] = torch.where(torch.arange(dim) % 3 == 0, 1.0, -1.0)  # unit RMS
    x[4] = 1e15 * torch.linspace(-1, 1, dim)       # large magnitudes
    x[5] = 1e-12 * torch.linspace(-1, 1, dim)      # small magnitudes (eps dominates)
    xb = x.to(torch.bfloat16)
    eps = 1e-6
    y = na.rms_norm(xb.cuda(), None, eps)
    torch.cuda.synchronize()
    _compare(y, xb, None, eps, "special rows")
    yc = y.float().cpu()
    assert torch.all(yc[0] == 0)                   # zero row stays zero
    assert torch.all(yc[3].abs() == torch.tensor(1.0 / np.sqrt(1.0 + eps)).to(torch.bfloat16).float())


def test_no_weight_equals_unit_weight():
    torch = _torch()
    import neighborhood_attention_amd as na
    from na3d_inputs import make_norm_inputs

    x, _ = make_norm_inputs(200, 1032, 9, "cuda")
    ones = torch.ones(1032, dtype=torch.bfloat16, device="cuda")
    assert torch.equal(na.rms_norm(x, None), na.rms_norm(x, ones))


def test_leading_axes_and_empty():
    torch = _torch()
    import neighborhood_attention_amd as na
    from na3d_inputs import make_norm_inputs

    x, w = make_norm_inputs(2 * 3 * 5, 264, 10, "cuda")
    y3 = na.rms_norm(x.view(2, 3, 5, 264), w)
    assert y3.shape == (2, 3, 5, 264)
    assert torch.equal(y3.view(30, 264), na.rms_norm(x, w))
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert na.rms_norm(e, None).shape == (0, 64)


def test_bad_arguments_raise():
    torch = _torch()
    import neighborhood_attention_amd as na

    x = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(na.NA3DError):
        na.rms_norm(x)                             # dim not a multiple of 8
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(na.NA3DError):
        na.rms_norm(x, eps=-1.0)
    with pytest.raises(ValueError):
        na.rms_norm(x, torch.ones(32, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        na.rms_norm(x.t())                         # not contiguous


def test_full_size_block_norm():
    """The benchmark's workload at full size, in its launch configuration,
    compared with the oracle on every element."""
    torch = _torch()
    import neighborhood_attention_amd as na
    from na3d_inputs import NORM_WORKLOADS, make_norm_inputs

    wl = NORM_WORKLOADS["rms_block_norm"]
    x, w = make_norm_inputs(wl.rows, wl.dim, wl.seed, "cuda")
    y = na.rms_norm(x, w, 1e-6)
    torch.cuda.synchronize()
    for lo in range(0, wl.rows, 4096):             # in slices to bound host memory
        sl = slice(lo, lo + 4096)
        _compare(y[sl], x[sl], w, 1e-6, "rows %d.." % lo)
