"""torch.library registrations of the library's entry points, and an RMSNorm
module, so that torch.compile and graph capture see them as opaque
functional ops.

The xDiT PR "LTX-2.5 optimizations: add parallel VAE decoding and AITER
RMSNorm" (Changes, item 2) wraps its bf16 RMSNorm kernel as a custom op that
declares no mutated arguments, because a wrongly declared mutation made
torch.compile skip graph capture at every call site, and swaps a drop-in
module (with or without an elementwise weight) into the model's block
norms.  The same shape is given here:

    y = torch.ops.na3d_amd.rms_norm(x, weight, eps)      # weight may be None
    o = torch.ops.na3d_amd.na3d_fwd(q, k, v, [KT, KH, KW])
    norm = RMSNorm(4096, eps=1e-6, elementwise_affine=True)

Each op allocates its output and calls the C ABI; nothing else happens
here.  The fake (meta) implementations give torch.compile the output shape
without running anything.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import fwd as _fwd
from . import rms_norm as _rms_norm


@torch.library.custom_op("na3d_amd::rms_norm", mutates_args=())
def rms_norm(x: torch.Tensor, weight: Optional[torch.Tensor], eps: float) -> torch.Tensor:
    return _rms_norm(x.contiguous(), weight, float(eps))


@rms_norm.register_fake
def _rms_norm_fake(x, weight, eps):
    return torch.empty_like(x, memory_format=torch.contiguous_format)


@torch.library.custom_op("na3d_amd::na3d_fwd", mutates_args=())
def na3d_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             kernel_size: List[int]) -> torch.Tensor:
    return _fwd(q, k, v, tuple(int(x) for x in kernel_size))


@na3d_fwd.register_fake
def _na3d_fwd_fake(q, k, v, kernel_size):
    return torch.empty(q.shape, dtype=q.dtype, device=q.device)


class RMSNorm(torch.nn.Module):
    """RMSNorm over the last axis on the HIP kernel: bf16 activations, an
    optional (dim,) weight (elementwise_affine=False: no weight, i.e. a unit
    one), eps added to the mean square."""

    def __init__(self, dim: int, eps: float = 1e-6, elementwise_affine: bool = True,
                 device=None):
        super().__init__()
        self.dim = int(dim)
        self.eps = float(eps)
        if elementwise_affine:
            # inference only (the op has no backward)
            self.weight = torch.nn.Parameter(
                torch.ones(self.dim, dtype=torch.bfloat16, device=device), requires_grad=False)
        else:
            self.register_parameter("weight", None)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return rms_norm(x, self.weight, self.eps)

    def extra_repr(self) -> str:
        return "%d, eps=%g, elementwise_affine=%s" % (self.dim, self.eps, self.weight is not None)
