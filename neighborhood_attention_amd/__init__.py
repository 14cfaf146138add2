"""Python binding of the MI355X NA3D forward library (``libna3d.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/na3d.h``.  torch supplies
device memory and the current stream.  There is no CPU or eager fallback:
if the library is missing or the device is not gfx950, calls raise.

    out = neighborhood_attention_amd.fwd(q, k, v, kernel_size=(3, 7, 7))

mirrors ``na3d_flash_attn(q, k, v, kernel_size)`` of the ROCm/aiter PR
"Add 3D neighborhood flash attention (na3d_flash)" (Technical Details):
(B, T, H, W, NH, HD) bf16 tensors, Q pre-scaled by head_dim**-0.5.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libna3d.so")

NA3D_OK = 0
NA3D_ERR_NULL = -1
NA3D_ERR_SHAPE = -2
NA3D_ERR_WINDOW = -3
NA3D_ERR_HEAD_DIM = -4
NA3D_ERR_ALIGN = -5
NA3D_ERR_OVERLAP = -6
NA3D_ERR_DEVICE = -7
NA3D_ERR_LAUNCH = -8
NA3D_ERR_CONFIG = -9
NA3D_ERR_STRIDE = -10
NA3D_ERR_BOX = -11
NA3D_ERR_VALUE = -12

EXPORTS = ("na3d_fwd", "na3d_check_args", "na3d_status_string", "na3d_plan",
           "na3d_fwd_config", "na3d_plan_config", "na3d_fwd_strided", "na3d_check_args_strided",
           "na3d_fwd_strided_config", "na3d_fwd_subgrid", "na3d_check_args_subgrid",
           "na3d_fwd_subgrid_config", "na3d_rms_norm", "na3d_check_args_rms_norm",
           "na3d_rms_norm_config", "na3d_fwd_batch", "na3d_check_args_batch",
           "na3d_plan_batch", "na3d_num_variants", "na3d_variant_info", "na3d_abi_version")
PLAN_KEYS = ("family", "tile_t", "tile_h", "tile_w", "workgroups", "threads", "lds_bytes",
             "planes", "variant", "runs")

_lock = threading.Lock()
_lib = None


class Tile(ctypes.Structure):
    """``na3d_tile``: one grid of a batch (device addresses and sizes)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("B", ctypes.c_int), ("T", ctypes.c_int),
                ("H", ctypes.c_int), ("W", ctypes.c_int)]


class NA3DError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def load(path: str = LIB_PATH):
    """Load (building first if absent) and type the C ABI."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            from . import _build
            _build.build()
        lib = ctypes.CDLL(path)
        i32, p = ctypes.c_int, ctypes.c_void_p
        lib.na3d_fwd.argtypes = [p, p, p, p] + [i32] * 9 + [p]
        lib.na3d_fwd.restype = i32
        lib.na3d_check_args.argtypes = [p, p, p, p] + [i32] * 9
        lib.na3d_check_args.restype = i32
        lib.na3d_status_string.argtypes = [i32]
        lib.na3d_status_string.restype = ctypes.c_char_p
        lib.na3d_plan.argtypes = [i32] * 9 + [ctypes.POINTER(i32)]
        lib.na3d_plan.restype = i32
        lib.na3d_fwd_config.argtypes = [p, p, p, p] + [i32] * 12 + [p]
        lib.na3d_fwd_config.restype = i32
        lib.na3d_plan_config.argtypes = [i32] * 12 + [ctypes.POINTER(i32)]
        lib.na3d_plan_config.restype = i32
        ll = ctypes.POINTER(ctypes.c_longlong)
        lib.na3d_fwd_strided.argtypes = [p, p, p, p] + [i32] * 9 + [ll, p]
        lib.na3d_fwd_strided.restype = i32
        lib.na3d_check_args_strided.argtypes = [p, p, p, p] + [i32] * 9 + [ll]
        lib.na3d_check_args_strided.restype = i32
        lib.na3d_fwd_strided_config.argtypes = [p, p, p, p] + [i32] * 9 + [ll] + [i32] * 3 + [p]
        lib.na3d_fwd_strided_config.restype = i32
        ip = ctypes.POINTER(i32)
        lib.na3d_fwd_subgrid.argtypes = [p, p, p, p] + [i32] * 9 + [ip, ll, p]
        lib.na3d_fwd_subgrid.restype = i32
        lib.na3d_check_args_subgrid.argtypes = [p, p, p, p] + [i32] * 9 + [ip, ll]
        lib.na3d_check_args_subgrid.restype = i32
        lib.na3d_fwd_subgrid_config.argtypes = [p, p, p, p] + [i32] * 9 + [ip, ll] + [i32] * 3 + [p]
        lib.na3d_fwd_subgrid_config.restype = i32
        f32 = ctypes.c_float
        lib.na3d_rms_norm.argtypes = [p, p, p, i32, i32, f32, p]
        lib.na3d_rms_norm.restype = i32
        lib.na3d_check_args_rms_norm.argtypes = [p, p, p, i32, i32, f32]
        lib.na3d_check_args_rms_norm.restype = i32
        lib.na3d_rms_norm_config.argtypes = [p, p, p, i32, i32, f32, i32, p]
        lib.na3d_rms_norm_config.restype = i32
        tp = ctypes.POINTER(Tile)
        lib.na3d_fwd_batch.argtypes = [tp, i32] + [i32] * 5 + [p]
        lib.na3d_fwd_batch.restype = i32
        lib.na3d_check_args_batch.argtypes = [tp, i32] + [i32] * 5
        lib.na3d_check_args_batch.restype = i32
        lib.na3d_plan_batch.argtypes = [tp, i32] + [i32] * 5 + [ctypes.POINTER(i32)]
        lib.na3d_plan_batch.restype = i32
        lib.na3d_num_variants.argtypes = []
        lib.na3d_num_variants.restype = i32
        lib.na3d_variant_info.argtypes = [i32, ctypes.POINTER(i32)]
        lib.na3d_variant_info.restype = i32
        lib.na3d_abi_version.argtypes = []
        lib.na3d_abi_version.restype = i32
        _lib = lib
        return lib


def _on_device(dev, call):
    """Run call(stream) with dev current and its current stream; the device
    switch is skipped when dev already is the current device."""
    import torch

    if dev.index is None or dev.index == torch.cuda.current_device():
        return call(torch.cuda.current_stream(dev).cuda_stream)
    with torch.cuda.device(dev):
        return call(torch.cuda.current_stream(dev).cuda_stream)


def status_string(status: int) -> str:
    return load().na3d_status_string(int(status)).decode()


def check_args(q_ptr, k_ptr, v_ptr, out_ptr, shape, kernel_size) -> int:
    """Host-only argument check on raw addresses (no device access)."""
    B, T, H, W, NH, HD = (int(x) for x in shape)
    KT, KH, KW = (int(x) for x in kernel_size)
    return load().na3d_check_args(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD,
                                  KT, KH, KW)


def _stride_array(strides):
    """20 element strides (B, T, H, W, NH of q, k, v, out) as a C array."""
    flat = [int(x) for group in strides for x in group]
    if len(flat) != 20:
        raise ValueError("expected 4 groups of 5 strides, got %d values" % len(flat))
    return (ctypes.c_longlong * 20)(*flat)


def check_args_strided(q_ptr, k_ptr, v_ptr, out_ptr, shape, kernel_size, strides) -> int:
    """Host-only argument check of the strided entry point (no device access).
    ``strides`` = four (sB, sT, sH, sW, sN) element-stride tuples: q, k, v, out."""
    B, T, H, W, NH, HD = (int(x) for x in shape)
    KT, KH, KW = (int(x) for x in kernel_size)
    return load().na3d_check_args_strided(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD,
                                          KT, KH, KW, _stride_array(strides))


def check_args_subgrid(q_ptr, k_ptr, v_ptr, out_ptr, shape, kernel_size, box, strides=None) -> int:
    """Host-only argument check of the query-box entry point.  ``shape`` is the
    k/v grid, ``box`` = (t0, h0, w0, Tq, Hq, Wq), ``strides`` as for
    check_args_strided or None for contiguous tensors."""
    B, T, H, W, NH, HD = (int(x) for x in shape)
    KT, KH, KW = (int(x) for x in kernel_size)
    bx = (ctypes.c_int * 6)(*[int(x) for x in box])
    st = None if strides is None else _stride_array(strides)
    return load().na3d_check_args_subgrid(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD,
                                          KT, KH, KW, bx, st)


def plan(shape, kernel_size, family: int = 0, variant: int = 0, tile_t: int = 0) -> dict:
    """Launch plan for these sizes (automatic, or an explicit configuration)."""
    B, T, H, W, NH, HD = (int(x) for x in shape)
    KT, KH, KW = (int(x) for x in kernel_size)
    buf = (ctypes.c_int * 10)()
    rc = load().na3d_plan_config(B, T, H, W, NH, HD, KT, KH, KW, int(family), int(variant),
                                 int(tile_t), buf)
    if rc != NA3D_OK:
        raise NA3DError(rc, "na3d_plan")
    return dict(zip(PLAN_KEYS, list(buf)))


def num_variants() -> int:
    return int(load().na3d_num_variants())


VARIANT_FIELDS = ("hd", "qh", "qw", "wh", "wt", "ns", "nk", "ng", "nbuf", "occ")


def variant_info(variant: int) -> dict:
    """Compile-time shape of a rolling instantiation (na3d_variant_info):
    head dim, query block QH x QW on each of 16 / (QH*QW) planes, wave grid,
    slots, tiles per group, groups, plane buffers, occupancy cap."""
    buf = (ctypes.c_int * 10)()
    rc = load().na3d_variant_info(int(variant), buf)
    if rc != NA3D_OK:
        raise NA3DError(rc, "na3d_variant_info")
    return dict(zip(VARIANT_FIELDS, (int(x) for x in buf)))


def fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, shape, kernel_size,
            stream: int = 0, config=None, strides=None, box=None) -> None:
    """Call na3d_fwd (or na3d_fwd_config when ``config`` = (family, variant,
    tile_t) is given; the strided entry points when ``strides`` = four
    (sB, sT, sH, sW, sN) element-stride tuples for q, k, v, out is given) on
    raw device addresses; raises NA3DError on failure."""
    B, T, H, W, NH, HD = (int(x) for x in shape)
    KT, KH, KW = (int(x) for x in kernel_size)
    if box is not None:
        bx = (ctypes.c_int * 6)(*[int(x) for x in box])
        st = None if strides is None else _stride_array(strides)
        fam, var, tt = (0, 0, 0) if config is None else (int(x) for x in config)
        rc = load().na3d_fwd_subgrid_config(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD,
                                            KT, KH, KW, bx, st, fam, var, tt, stream)
    elif strides is not None:
        st = _stride_array(strides)
        if config is None:
            rc = load().na3d_fwd_strided(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD, KT,
                                         KH, KW, st, stream)
        else:
            fam, var, tt = (int(x) for x in config)
            rc = load().na3d_fwd_strided_config(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH,
                                                HD, KT, KH, KW, st, fam, var, tt, stream)
    elif config is None:
        rc = load().na3d_fwd(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD, KT, KH, KW,
                             stream)
    else:
        fam, var, tt = (int(x) for x in config)
        rc = load().na3d_fwd_config(q_ptr, k_ptr, v_ptr, out_ptr, B, T, H, W, NH, HD, KT,
                                    KH, KW, fam, var, tt, stream)
    if rc != NA3D_OK:
        raise NA3DError(rc, "na3d_fwd")


def fwd(q, k, v, kernel_size, out=None, config=None):
    """3-D neighborhood attention forward on (B,T,H,W,NH,HD) bf16 CUDA tensors.

    q, k, v (and out) may be strided views, e.g. slices of a fused QKV
    projection output, as long as the HD axis is contiguous; they are then
    read in place through na3d_fwd_strided.  Returns ``out`` (a new
    contiguous tensor when not given).  The kernel is enqueued on torch's
    current stream.  ``config`` = (family, variant, tile_t) forces a launch
    configuration (tuning/testing).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
        if t.device.type != "cuda":
            raise ValueError("%s must be a GPU tensor" % name)
        if t.dim() == 6 and t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("%s must have a contiguous last (head-dim) axis" % name)
    if q.dim() != 6:
        raise ValueError("expected (B,T,H,W,NH,HD) tensors, got %d dims" % q.dim())
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ: %s %s %s" % (q.shape, k.shape, v.shape))
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    elif (out.shape != q.shape or out.dtype != torch.bfloat16 or out.device != q.device
          or (out.shape[-1] > 1 and out.stride(-1) != 1)):
        raise ValueError("out must be a bf16 tensor shaped like q with a contiguous last axis")
    tensors = (q, k, v, out)
    strides = None
    if not all(t.is_contiguous() for t in tensors):
        strides = [tuple(int(x) for x in t.stride()[:5]) for t in tensors]
    _on_device(q.device, lambda stream: fwd_raw(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), q.shape, kernel_size, stream,
        config, strides))
    return out


def fwd_subgrid(q, k, v, kernel_size, offset, out=None, config=None):
    """Neighborhood attention for the queries of a sub-box of the grid, with
    windows placed in the whole grid.

    k, v: (B,T,H,W,NH,HD), the whole grid.  q (and out): (B,Tq,Hq,Wq,NH,HD),
    the queries at grid positions offset + (i, j, l), offset = (t0, h0, w0).
    The result equals the same box of ``fwd`` over the whole grid.  Strided
    views are accepted as in ``fwd``.  Returns ``out``.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device.type != "cuda":
            raise TypeError("%s must be a bfloat16 GPU tensor" % name)
        if t.dim() != 6:
            raise ValueError("expected (B,T,H,W,NH,HD) tensors, got %d dims for %s" % (t.dim(), name))
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("%s must have a contiguous last (head-dim) axis" % name)
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ: %s %s" % (k.shape, v.shape))
    if q.shape[0] != k.shape[0] or q.shape[4:] != k.shape[4:]:
        raise ValueError("q %s does not match the batch/heads/head dim of k %s" % (q.shape, k.shape))
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")
    t0, h0, w0 = (int(x) for x in offset)
    box = (t0, h0, w0, q.shape[1], q.shape[2], q.shape[3])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    elif (out.shape != q.shape or out.dtype != torch.bfloat16 or out.device != q.device
          or (out.shape[-1] > 1 and out.stride(-1) != 1)):
        raise ValueError("out must be a bf16 tensor shaped like q with a contiguous last axis")
    tensors = (q, k, v, out)
    strides = None
    if not all(t.is_contiguous() for t in tensors):
        strides = [tuple(int(x) for x in t.stride()[:5]) for t in tensors]
    _on_device(q.device, lambda stream: fwd_raw(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), k.shape, kernel_size, stream,
        config, strides, box))
    return out


def check_args_rms_norm(x_ptr, w_ptr, y_ptr, rows, dim, eps) -> int:
    """Host-only argument check of na3d_rms_norm (no device access)."""
    return load().na3d_check_args_rms_norm(x_ptr, w_ptr, y_ptr, int(rows), int(dim), float(eps))


def rms_norm_raw(x_ptr: int, w_ptr, y_ptr: int, rows: int, dim: int, eps: float,
                 stream: int = 0, workgroups=None) -> None:
    """Call na3d_rms_norm (na3d_rms_norm_config when ``workgroups`` is given)
    on raw device addresses; ``w_ptr`` None or 0 means a unit weight."""
    w_ptr = w_ptr or None
    if workgroups is None:
        rc = load().na3d_rms_norm(x_ptr, w_ptr, y_ptr, int(rows), int(dim), float(eps), stream)
    else:
        rc = load().na3d_rms_norm_config(x_ptr, w_ptr, y_ptr, int(rows), int(dim), float(eps),
                                         int(workgroups), stream)
    if rc != NA3D_OK:
        raise NA3DError(rc, "na3d_rms_norm")


def rms_norm(x, weight=None, eps: float = 1e-6, out=None, workgroups=None):
    """RMSNorm over the last axis of a contiguous bf16 GPU tensor:
    x * weight / sqrt(mean(x**2, -1) + eps), fp32 inside, one bf16 rounding.

    The drop-in block norm of the xDiT PR "LTX-2.5 optimizations: add
    parallel VAE decoding and AITER RMSNorm" (Changes, item 2): ``weight``
    (shape (dim,), bf16) or None for a norm without an elementwise weight.
    ``out`` may be ``x`` itself (in place).  Enqueued on torch's current
    stream.  ``workgroups`` forces the grid size (tuning/testing).
    """
    import torch

    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.device.type != "cuda":
        raise TypeError("x must be a bfloat16 GPU tensor")
    if x.dim() < 1 or not x.is_contiguous():
        raise ValueError("x must be a contiguous tensor with at least one axis")
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    if weight is not None:
        if (not isinstance(weight, torch.Tensor) or weight.dtype != torch.bfloat16
                or weight.device != x.device or tuple(weight.shape) != (dim,)
                or not weight.is_contiguous()):
            raise ValueError("weight must be a contiguous bf16 (dim,) tensor on x's device")
    if out is None:
        out = torch.empty_like(x)
    elif (out.shape != x.shape or out.dtype != torch.bfloat16 or out.device != x.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 tensor shaped like x")
    _on_device(x.device, lambda stream: rms_norm_raw(
        x.data_ptr(), None if weight is None else weight.data_ptr(), out.data_ptr(), rows, dim,
        eps, stream, workgroups))
    return out


def _tile_array(tiles):
    """tiles: sequence of (q_ptr, k_ptr, v_ptr, out_ptr, (B, T, H, W))."""
    arr = (Tile * max(len(tiles), 1))()
    for i, (q, k, v, o, dims) in enumerate(tiles):
        B, T, H, W = (int(x) for x in dims)
        arr[i] = Tile(q, k, v, o, B, T, H, W)
    return arr


def check_args_batch(tiles, NH, HD, kernel_size) -> int:
    """Host-only check of a batch given as (q_ptr, k_ptr, v_ptr, out_ptr,
    (B, T, H, W)) tuples (no device access)."""
    KT, KH, KW = (int(x) for x in kernel_size)
    return load().na3d_check_args_batch(_tile_array(tiles), len(tiles), int(NH), int(HD),
                                        KT, KH, KW)


def plan_batch(dims, NH, HD, kernel_size) -> dict:
    """How a batch of grids of the given (B, T, H, W) sizes would be launched."""
    KT, KH, KW = (int(x) for x in kernel_size)
    arr = _tile_array([(0, 0, 0, 0, d) for d in dims])
    buf = (ctypes.c_int * 4)()
    rc = load().na3d_plan_batch(arr, len(dims), int(NH), int(HD), KT, KH, KW, buf)
    if rc != NA3D_OK:
        raise NA3DError(rc, "na3d_plan_batch")
    return dict(zip(("launches", "variant", "shared_tiles", "workgroups"), list(buf)))


def fwd_batch_raw(tiles, NH, HD, kernel_size, stream: int = 0) -> None:
    KT, KH, KW = (int(x) for x in kernel_size)
    rc = load().na3d_fwd_batch(_tile_array(tiles), len(tiles), int(NH), int(HD), KT, KH, KW,
                               stream)
    if rc != NA3D_OK:
        raise NA3DError(rc, "na3d_fwd_batch")


def fwd_batch(qkv, kernel_size, outs=None):
    """NA3D forward on many independent grids (e.g. the tiles of a decoder's
    tile grid) in as few launches as possible.

    qkv: sequence of (q, k, v) triples of contiguous (B,T,H,W,NH,HD) bf16 GPU
    tensors; every triple may have its own B, T, H, W; NH, HD and the window
    are shared.  Returns the list of outputs (new tensors unless ``outs`` is
    given); each equals ``fwd`` on its triple alone.
    """
    import torch

    qkv = list(qkv)
    if not qkv:
        return []
    dev = qkv[0][0].device
    NH, HD = qkv[0][0].shape[4], qkv[0][0].shape[5]
    for i, trip in enumerate(qkv):
        if len(trip) != 3:
            raise ValueError("entry %d is not a (q, k, v) triple" % i)
        for t in trip:
            if (not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device != dev
                    or t.dim() != 6 or not t.is_contiguous()):
                raise ValueError("entry %d: q, k, v must be contiguous 6-d bf16 tensors on %s"
                                 % (i, dev))
        if not (trip[0].shape == trip[1].shape == trip[2].shape):
            raise ValueError("entry %d: q, k, v shapes differ" % i)
        if trip[0].shape[4] != NH or trip[0].shape[5] != HD:
            raise ValueError("entry %d: every tile must have NH=%d and HD=%d" % (i, NH, HD))
    if outs is None:
        outs = [torch.empty_like(trip[0]) for trip in qkv]
    elif len(outs) != len(qkv) or any(
            o.shape != t[0].shape or o.dtype != torch.bfloat16 or o.device != dev
            or not o.is_contiguous() for o, t in zip(outs, qkv)):
        raise ValueError("outs must be contiguous bf16 tensors shaped like each q")
    tiles = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), q.shape[:4])
             for (q, k, v), o in zip(qkv, outs)]
    _on_device(dev, lambda stream: fwd_batch_raw(tiles, NH, HD, kernel_size, stream))
    return outs
