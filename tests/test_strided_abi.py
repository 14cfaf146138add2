"""Host-only checks of the strided entry point's contract (no GPU needed):
the strides that na3d_fwd_strided accepts and the ones it rejects before any
device call."""
import pytest

import neighborhood_attention_amd as na

SHAPE = (2, 4, 6, 8, 2, 32)
KS = (3, 5, 5)
BASE = 0x100000


def contiguous(shape):
    B, T, H, W, NH, HD = shape
    sn = HD
    sw = NH * HD
    sh = W * sw
    st = H * sh
    sb = T * st
    return (sb, st, sh, sw, sn)


def fused(shape, inner):
    """Strides of q/k/v sliced out of a fused QKV buffer: inner=False puts the
    3 before NH (B,T,H,W,3,NH,HD), inner=True after it (B,T,H,W,NH,3,HD)."""
    B, T, H, W, NH, HD = shape
    tok = 3 * NH * HD
    sn = 3 * HD if inner else HD
    return (T * H * W * tok, H * W * tok, W * tok, tok, sn)


def nbytes(shape):
    n = 2
    for x in shape:
        n *= x
    return n


def check(ptrs, strides, shape=SHAPE, ks=KS):
    return na.check_args_strided(*ptrs, shape, ks, strides)


def test_contiguous_strides_match_plain_check():
    c = contiguous(SHAPE)
    n = nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    assert check(ptrs, [c] * 4) == na.NA3D_OK
    assert na.check_args(*ptrs, SHAPE, KS) == na.NA3D_OK


@pytest.mark.parametrize("inner", [False, True])
def test_fused_qkv_views_pass(inner):
    s = fused(SHAPE, inner)
    n3 = 3 * nbytes(SHAPE)
    step = 2 * (SHAPE[5] if inner else SHAPE[4] * SHAPE[5])  # bytes between the q, k, v slices
    ptrs = (BASE, BASE + step, BASE + 2 * step, BASE + n3)
    assert check(ptrs, [s, s, s, contiguous(SHAPE)]) == na.NA3D_OK


def test_head_major_views_pass():
    B, T, H, W, NH, HD = SHAPE
    s = (NH * T * H * W * HD, H * W * HD, W * HD, HD, T * H * W * HD)
    n = nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    assert check(ptrs, [s, s, s, s]) == na.NA3D_OK


def test_padded_output_passes():
    B, T, H, W, NH, HD = SHAPE
    so = contiguous((B, T, H, W, NH, HD + 16))
    n = nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    assert check(ptrs, [contiguous(SHAPE)] * 3 + [so]) == na.NA3D_OK


@pytest.mark.parametrize("tensor", range(4))
@pytest.mark.parametrize("axis", range(5))
def test_negative_or_unaligned_stride(tensor, axis):
    n = nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    for bad in (-contiguous(SHAPE)[axis], contiguous(SHAPE)[axis] + 4):
        st = [list(contiguous(SHAPE)) for _ in range(4)]
        st[tensor][axis] = bad
        assert check(ptrs, st) == na.NA3D_ERR_STRIDE


@pytest.mark.parametrize("axis", [2, 3, 4])
def test_k_and_v_must_share_spatial_and_head_strides(axis):
    n = 4 * nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    sv = list(contiguous(SHAPE))
    sv[axis] *= 2
    assert check(ptrs, [contiguous(SHAPE), contiguous(SHAPE), sv, contiguous(SHAPE)]) == \
        na.NA3D_ERR_STRIDE


def test_k_and_v_may_differ_in_batch_and_plane_strides():
    n = 4 * nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    sv = list(contiguous(SHAPE))
    sv[0] *= 2
    sv[1] *= 2
    assert check(ptrs, [contiguous(SHAPE), contiguous(SHAPE), sv, contiguous(SHAPE)]) == na.NA3D_OK


def test_output_that_maps_two_elements_to_one_address():
    n = nbytes(SHAPE)
    ptrs = (BASE, BASE + n, BASE + 2 * n, BASE + 3 * n)
    so = list(contiguous(SHAPE))
    so[3] = 0                      # every w of a row on one address
    assert check(ptrs, [contiguous(SHAPE)] * 3 + [so]) == na.NA3D_ERR_STRIDE
    so = list(contiguous(SHAPE))
    so[4] = 16                     # heads 16 elements apart, HD = 32: overlapping rows
    assert check(ptrs, [contiguous(SHAPE)] * 3 + [so]) == na.NA3D_ERR_STRIDE
    # extent-1 axes may have any stride
    one = (1,) + SHAPE[1:]
    so = list(contiguous(one))
    so[0] = 0
    assert check(ptrs, [contiguous(one)] * 3 + [so], shape=one) == na.NA3D_OK


def test_output_inside_a_fused_input_is_rejected():
    s = fused(SHAPE, False)
    step = 2 * SHAPE[4] * SHAPE[5]
    ptrs = (BASE, BASE + step, BASE + 2 * step, BASE + 3 * nbytes(SHAPE) - 64)
    assert check(ptrs, [s, s, s, contiguous(SHAPE)]) == na.NA3D_ERR_OVERLAP


def test_null_strides_and_pointers():
    lib = na.load()
    n = nbytes(SHAPE)
    assert lib.na3d_check_args_strided(BASE, BASE + n, BASE + 2 * n, BASE + 3 * n, *SHAPE, *KS,
                                       None) == na.NA3D_ERR_NULL
    assert check((0, BASE + n, BASE + 2 * n, BASE + 3 * n), [contiguous(SHAPE)] * 4) == \
        na.NA3D_ERR_NULL


def test_strided_fwd_rejects_before_any_device_call():
    lib = na.load()
    n = nbytes(SHAPE)
    st = na._stride_array([contiguous(SHAPE)] * 3 + [(0, 0, 0, 0, 0)])
    assert lib.na3d_fwd_strided(BASE, BASE + n, BASE + 2 * n, BASE + 3 * n, *SHAPE, *KS, st,
                                None) == na.NA3D_ERR_STRIDE
    assert lib.na3d_fwd_strided_config(BASE, BASE + n, BASE + 2 * n, BASE + 3 * n, *SHAPE, *KS,
                                       st, 2, 0, 0, None) == na.NA3D_ERR_STRIDE


def test_stride_array_shape():
    with pytest.raises(ValueError):
        na._stride_array([(1, 2, 3, 4, 5)] * 3)


def test_stride_products_that_overflow_are_rejected():
    """Strides up to 2^56 times extents up to 2^31 exceed 64 bits: the span
    and extent arithmetic must report them, not wrap."""
    shape = (1 << 20, 4, 6, 8, 2, 32)
    c = contiguous(SHAPE)
    huge = (1 << 56, c[1], c[2], c[3], c[4])
    ptrs = (BASE, BASE + (1 << 40), BASE + (2 << 40), BASE + (3 << 40))
    assert check(ptrs, [huge, c, c, c], shape=shape) == na.NA3D_ERR_STRIDE
    assert check(ptrs, [c, c, c, huge], shape=shape) == na.NA3D_ERR_STRIDE
    assert check(ptrs, [c, huge, huge, c], shape=shape) == na.NA3D_ERR_STRIDE
