"""Host-side contract of the RMSNorm entry points (no GPU needed): the
argument checks reject bad sizes, eps, alignment and overlaps before any
device call."""
import math

import pytest

import neighborhood_attention_amd as na

X, W, Y = 0x100000, 0x20000000, 0x40000000  # fake 16-B aligned addresses


def check(x=X, w=W, y=Y, rows=64, dim=4096, eps=1e-6):
    return na.check_args_rms_norm(x, w, y, rows, dim, eps)


def test_valid_arguments_pass():
    assert check() == na.NA3D_OK
    assert check(w=0) == na.NA3D_OK                      # no weight: unit weight
    assert check(rows=0) == na.NA3D_OK                   # empty input is a no-op
    assert check(x=0, w=0, y=0, rows=0) == na.NA3D_OK    # (an empty tensor has no address)
    assert check(x=0, y=0, rows=0, dim=12) == na.NA3D_ERR_SHAPE
    assert check(dim=8, rows=1) == na.NA3D_OK
    assert check(dim=8192) == na.NA3D_OK
    assert check(eps=0.0) == na.NA3D_OK
    assert check(y=X) == na.NA3D_OK                      # in place


@pytest.mark.parametrize("which", ["x", "y"])
def test_null_tensor(which):
    assert check(**{which: 0}) == na.NA3D_ERR_NULL


@pytest.mark.parametrize("rows,dim", [(-1, 64), (4, 0), (4, 4), (4, 12), (4, 8200),
                                      (4, 16384), (4, -8)])
def test_bad_sizes(rows, dim):
    assert check(rows=rows, dim=dim) == na.NA3D_ERR_SHAPE


@pytest.mark.parametrize("eps", [-1e-6, -1.0, math.inf, -math.inf, math.nan])
def test_bad_eps(eps):
    assert check(eps=eps) == na.NA3D_ERR_VALUE


@pytest.mark.parametrize("which", ["x", "w", "y"])
def test_misaligned(which):
    base = {"x": X, "w": W, "y": Y}[which]
    assert check(**{which: base + 8}) == na.NA3D_ERR_ALIGN


def test_overlaps():
    n = 64 * 4096 * 2
    assert check(y=X + 16) == na.NA3D_ERR_OVERLAP           # y shifted into x
    assert check(y=X + n - 16) == na.NA3D_ERR_OVERLAP
    assert check(y=X - n + 16) == na.NA3D_ERR_OVERLAP
    assert check(y=X + n) == na.NA3D_OK                     # adjacent, no overlap
    assert check(y=X - n) == na.NA3D_OK
    assert check(w=Y + n - 16) == na.NA3D_ERR_OVERLAP       # weight inside y
    assert check(w=Y - 4096 * 2 + 16) == na.NA3D_ERR_OVERLAP
    assert check(w=Y - 4096 * 2) == na.NA3D_OK
    assert check(w=X) == na.NA3D_OK                         # weight may alias x (both read)


def test_status_string_of_value_error():
    assert "eps" in na.status_string(na.NA3D_ERR_VALUE)


def test_config_rejects_bad_grid_without_device():
    lib = na.load()
    assert lib.na3d_rms_norm_config(X, W, Y, 64, 4096, 1e-6, -1, None) == na.NA3D_ERR_CONFIG
    assert lib.na3d_rms_norm_config(X, W, Y, 64, 4096, 1e-6, (1 << 24) + 1, None) == \
        na.NA3D_ERR_CONFIG
    # argument errors come first and never touch a device
    assert lib.na3d_rms_norm(X, W, Y, 64, 12, 1e-6, None) == na.NA3D_ERR_SHAPE
    assert lib.na3d_rms_norm(X, W, Y, 0, 4096, 1e-6, None) == na.NA3D_OK


def test_python_wrapper_type_checks():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        na.rms_norm(torch.zeros(4, 8, dtype=torch.bfloat16))          # CPU tensor
    with pytest.raises(TypeError):
        na.rms_norm([1.0, 2.0])
