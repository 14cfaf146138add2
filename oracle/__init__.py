"""CPU oracle for the NA3D forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package.  The product library
(``neighborhood_attention_amd``) never imports it, and the two share no code.

The arithmetic lives in ``na3d_oracle.c`` (plain C, double precision, fixed
summation order); this module only compiles it with gcc and marshals numpy
arrays through ctypes.  What is computed follows the ROCm/aiter PR page
"Add 3D neighborhood flash attention (na3d_flash)", sections *Motivation*
(each token attends to its KT x KH x KW neighbours) and *Technical Details*
(inward border shift so every window holds exactly KT*KH*KW keys; (B,T,H,W,NH,HD)
bf16 tensors; Q pre-scaled by head_dim**-0.5).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "na3d_oracle.c")
_LIB = os.path.join(_HERE, "libna3d_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no FMA contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            i32, i64, p = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
            lib.na3d_oracle_window_start.argtypes = [i32, i32, i32]
            lib.na3d_oracle_window_start.restype = i32
            lib.na3d_oracle_max_threads.argtypes = [i32]
            lib.na3d_oracle_max_threads.restype = i32
            lib.na3d_oracle_fwd.argtypes = [p, p, p, p] + [i32] * 10
            lib.na3d_oracle_fwd.restype = i32
            lib.na3d_oracle_fwd_points.argtypes = [p, p, p, p, i64, p] + [i32] * 10
            lib.na3d_oracle_fwd_points.restype = i32
            lib.na3d_oracle_weights.argtypes = [p, p, p, p, p] + [i32] * 9
            lib.na3d_oracle_weights.restype = i32
            _lib = lib
    return _lib


def _as_bits(x) -> np.ndarray:
    """bf16 tensor (torch, CPU) or uint16 array -> contiguous uint16 bits."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("oracle expects bf16 bit patterns as uint16")
        return np.ascontiguousarray(x)
    import torch  # local: the oracle itself needs only numpy

    if x.dtype != torch.bfloat16:
        raise TypeError("oracle expects bfloat16 tensors")
    return x.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def _dims(q, kernel_size):
    if q.ndim != 6:
        raise ValueError("expected (B,T,H,W,NH,HD) tensors")
    kt, kh, kw = (int(x) for x in kernel_size)
    return tuple(int(s) for s in q.shape) + (kt, kh, kw)


def window_start(i: int, K: int, L: int) -> int:
    """clamp(i - K//2, 0, L - K); -1 for an undefined (i, K, L)."""
    return int(_load().na3d_oracle_window_start(int(i), int(K), int(L)))


def max_threads(nthreads: int = 0) -> int:
    return int(_load().na3d_oracle_max_threads(int(nthreads)))


def fwd(q, k, v, kernel_size, nthreads: int = 0) -> np.ndarray:
    """Full NA3D forward; returns a float64 (B,T,H,W,NH,HD) array."""
    qb, kb, vb = _as_bits(q), _as_bits(k), _as_bits(v)
    if not (qb.shape == kb.shape == vb.shape):
        raise ValueError("q, k, v shapes differ")
    dims = _dims(qb, kernel_size)
    out = np.empty(qb.shape, dtype=np.float64)
    rc = _load().na3d_oracle_fwd(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
                                 out.ctypes.data, *dims, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return out


def fwd_points(q, k, v, kernel_size, points, nthreads: int = 0) -> np.ndarray:
    """Outputs of selected queries; points is an (N,5) int array of (b,t,h,w,n).
    Returns an (N, HD) float64 array."""
    qb, kb, vb = _as_bits(q), _as_bits(k), _as_bits(v)
    if not (qb.shape == kb.shape == vb.shape):
        raise ValueError("q, k, v shapes differ")
    dims = _dims(qb, kernel_size)
    idx = np.ascontiguousarray(np.asarray(points, dtype=np.int64).reshape(-1, 5))
    out = np.empty((idx.shape[0], qb.shape[5]), dtype=np.float64)
    rc = _load().na3d_oracle_fwd_points(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
                                        idx.ctypes.data, idx.shape[0], out.ctypes.data,
                                        *dims, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return out


def weights(q, k, v, kernel_size):
    """Per-query softmax weights (B,T,H,W,NH,KT*KH*KW) in window order and the
    window starts (B,T,H,W,NH,3).  Tiny grids only."""
    qb, kb, vb = _as_bits(q), _as_bits(k), _as_bits(v)
    dims = _dims(qb, kernel_size)
    kt, kh, kw = dims[6:]
    w = np.empty(qb.shape[:5] + (kt * kh * kw,), dtype=np.float64)
    s = np.empty(qb.shape[:5] + (3,), dtype=np.int32)
    rc = _load().na3d_oracle_weights(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
                                     w.ctypes.data, s.ctypes.data, *dims)
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return w, s
