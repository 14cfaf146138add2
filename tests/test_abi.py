"""The C-ABI library loads, exports every symbol include/na3d.h declares,
and rejects bad arguments before touching any device (no GPU needed)."""
import ctypes
import os
import re

import pytest

import neighborhood_attention_amd as na

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "na3d.h")

A, B_, C, O = 0x10000, 0x20000000, 0x40000000, 0x60000000  # fake 16-B aligned addresses
SHAPE = (1, 4, 6, 8, 2, 32)
KS = (3, 5, 5)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(na3d_\w+)\s*\(", text, re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    assert {"na3d_fwd", "na3d_check_args", "na3d_status_string", "na3d_plan",
            "na3d_abi_version"} <= set(names)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(na.LIB_PATH if os.path.exists(na.LIB_PATH) else na.load()._name)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_python_binding_lists_all_exports():
    assert set(na.EXPORTS) == set(declared_functions())


def test_abi_version():
    assert na.load().na3d_abi_version() == 3


def test_variant_info():
    n = na.num_variants()
    assert n > 0
    for v in range(n):
        info = na.variant_info(v)
        assert info["hd"] in (16, 32, 64, 128, 256)
        assert info["qh"] * info["qw"] in (8, 16)          # 16 queries over 2 or 1 planes
        assert info["wh"] * info["wt"] * 64 <= 1024
        assert info["nbuf"] in (1, 2) and info["ns"] >= 1 and info["nk"] >= 1 and info["ng"] >= 1
    lib = na.load()
    buf = (ctypes.c_int * 10)()
    assert lib.na3d_variant_info(-1, buf) == na.NA3D_ERR_CONFIG
    assert lib.na3d_variant_info(n, buf) == na.NA3D_ERR_CONFIG
    assert lib.na3d_variant_info(0, None) == na.NA3D_ERR_NULL


def check(ptrs=(A, B_, C, O), shape=SHAPE, ks=KS):
    return na.check_args(*ptrs, shape, ks)


def test_valid_arguments_pass():
    assert check() == na.NA3D_OK
    assert check(shape=(2, 16, 64, 5, 8, 64), ks=(3, 5, 5)) == na.NA3D_OK
    assert check(shape=(1, 1, 1, 1, 1, 16), ks=(1, 1, 1)) == na.NA3D_OK
    assert check(shape=(1, 4, 6, 8, 2, 32), ks=(4, 6, 2)) == na.NA3D_OK  # even windows


@pytest.mark.parametrize("i", range(4))
def test_null_pointer(i):
    ptrs = [A, B_, C, O]
    ptrs[i] = 0
    assert check(ptrs=ptrs) == na.NA3D_ERR_NULL


@pytest.mark.parametrize("dim", range(6))
@pytest.mark.parametrize("val", [0, -3])
def test_bad_dimension(dim, val):
    shape = list(SHAPE)
    shape[dim] = val
    assert check(shape=shape) in (na.NA3D_ERR_SHAPE, na.NA3D_ERR_HEAD_DIM)


@pytest.mark.parametrize("ks", [(0, 5, 5), (3, 0, 5), (3, 5, -1), (5, 5, 5), (3, 7, 5), (3, 5, 9)])
def test_bad_window(ks):
    assert check(ks=ks) == na.NA3D_ERR_WINDOW


@pytest.mark.parametrize("hd", [8, 24, 48, 96, 512])
def test_unsupported_head_dim(hd):
    assert check(shape=SHAPE[:5] + (hd,)) == na.NA3D_ERR_HEAD_DIM


@pytest.mark.parametrize("hd", [16, 32, 64, 128, 256])
def test_supported_head_dims(hd):
    assert check(shape=SHAPE[:5] + (hd,)) == na.NA3D_OK


@pytest.mark.parametrize("i", range(4))
def test_misaligned_pointer(i):
    ptrs = [A, B_, C, O]
    ptrs[i] += 8
    assert check(ptrs=ptrs) == na.NA3D_ERR_ALIGN


def test_overlapping_output():
    nbytes = 1 * 4 * 6 * 8 * 2 * 32 * 2
    assert check(ptrs=(A, B_, C, A + nbytes - 16)) == na.NA3D_ERR_OVERLAP
    assert check(ptrs=(A, B_, C, C)) == na.NA3D_ERR_OVERLAP
    assert check(ptrs=(A, A, A, A + nbytes)) == na.NA3D_OK  # adjacent, q/k/v aliased


def test_oversized_grid():
    assert check(shape=(1, 2048, 2048, 2048, 1, 16), ks=(1, 1, 1)) == na.NA3D_ERR_SHAPE


def test_element_count_overflow_is_rejected():
    """A 2^69-element tensor whose count wraps to 0 in 64-bit arithmetic
    (B = 2^20, T = H = 2^10, W = 1, NH = 2^21, HD = 256) must not pass."""
    big = (1 << 20, 1 << 10, 1 << 10, 1, 1 << 21, 256)
    assert check(shape=big, ks=(1, 1, 1)) == na.NA3D_ERR_SHAPE
    assert na.load().na3d_fwd(A, B_, C, O, *big, 1, 1, 1, None) == na.NA3D_ERR_SHAPE
    assert check(shape=((1 << 31) - 1, 1, 1, 1, (1 << 31) - 1, 256), ks=(1, 1, 1)) \
        == na.NA3D_ERR_SHAPE


def test_status_strings():
    for code in range(0, -12, -1):
        s = na.status_string(code)
        assert s and s != "unknown status"
    assert na.status_string(-99) == "unknown status"


def test_fwd_rejects_before_any_device_call():
    lib = na.load()
    assert lib.na3d_fwd(0, B_, C, O, *SHAPE, *KS, None) == na.NA3D_ERR_NULL
    assert lib.na3d_fwd(A, B_, C, O, *SHAPE, 5, 5, 5, None) == na.NA3D_ERR_WINDOW
    assert lib.na3d_fwd(A + 2, B_, C, O, *SHAPE, *KS, None) == na.NA3D_ERR_ALIGN


def test_plan_covers_grid():
    for shape, ks in [((1, 16, 64, 96, 8, 64), (3, 7, 7)), ((1, 16, 64, 5, 8, 64), (3, 5, 5)),
                      ((1, 32, 128, 192, 16, 128), (3, 7, 7)), ((1, 16, 48, 64, 8, 64), (11, 11, 11))]:
        p = na.plan(shape, ks)
        B, T, H, W, NH, _ = shape
        tiles = p["runs"] * -(-H // p["tile_h"]) * -(-W // p["tile_w"])
        assert p["workgroups"] == B * NH * tiles
        assert 64 <= p["threads"] <= 1024 and p["threads"] % 64 == 0
        assert 0 < p["lds_bytes"] <= 160 * 1024
    with pytest.raises(na.NA3DError):
        na.plan((1, 2, 2, 2, 1, 32), (3, 1, 1))


def test_two_plane_tile_by_grid_length():
    """11x11x11 at head dim 64: two-plane blocks in 4-wave workgroups of
    4x4-query tiles on short grids, in 12-wave ones of 12x4-query tiles from
    32 query planes on."""
    for T, wh in [(16, 2), (24, 2), (32, 6), (79, 6)]:
        info = na.variant_info(na.plan((1, T, 96, 96, 8, 64), (11, 11, 11))["variant"])
        assert info["qh"] * info["qw"] == 8 and info["wh"] == wh, (T, info)


def test_head_dim_128_two_plane_workgroups():
    """Head dim 128, windows past the 2x8 7-tile variants: two-plane blocks in
    8-wave workgroups of 8x4-query tiles (two waves per SIMD); (5,7,7) stays
    on 2x8 blocks and the three-plane (3,7,7) on its staging-wave variant."""
    shape = (1, 16, 64, 96, 8, 128)
    for ks in [(11, 11, 11), (3, 11, 11), (7, 9, 9), (3, 7, 19)]:
        info = na.variant_info(na.plan(shape, ks)["variant"])
        assert (info["hd"], info["qh"] * info["qw"], info["wh"], info["wt"]) == (128, 8, 4, 2), ks
        assert na.plan(shape, ks)["threads"] == 512
    assert na.variant_info(na.plan(shape, (5, 7, 7))["variant"])["qw"] == 8
    assert na.plan(shape, (3, 7, 7))["threads"] == 768


def test_head_dim_128_wide_windows_eight_phases():
    """Head dim 128, windows whose 2x4-block union passes 11 tiles: 2x8
    blocks in two 9-tile groups, 8 waves along T (two waves per SIMD at the
    same 147 KB of LDS as the 4-wave form)."""
    for shape, ks in [((1, 16, 32, 32, 8, 128), (13, 13, 13)), ((1, 16, 64, 128, 8, 128), (3, 5, 27)),
                      ((1, 4, 8, 128, 32, 128), (3, 5, 35))]:
        info = na.variant_info(na.plan(shape, ks)["variant"])
        assert (info["hd"], info["qw"], info["wh"], info["wt"], info["ng"]) == (128, 8, 1, 8, 2), ks


def test_three_plane_tile_by_grid_size():
    """(3,7,7) at head dim 64: 12-wave 8x8-query tiles only on grids of 32 or
    more planes whose 8x8 tiles fill the chip without cutting the runs
    along T; 8-wave 4x8-query tiles otherwise."""
    for shape, rows in [((1, 16, 96, 128, 8, 64), 4), ((1, 31, 96, 128, 8, 64), 4),
                        ((1, 32, 96, 128, 8, 64), 8), ((1, 79, 192, 192, 8, 64), 8),
                        ((1, 64, 64, 96, 8, 64), 4), ((1, 33, 64, 96, 8, 64), 4)]:
        p = na.plan(shape, (3, 7, 7))
        assert (p["tile_h"], p["tile_w"]) == (rows, 8), (shape, p)
