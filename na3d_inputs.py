"""Seeded synthetic inputs for NA3D, shared by the tests, the smoke check and
the benchmark.

This module only draws random numbers; it holds none of the attention
arithmetic, and neither the oracle nor the GPU library imports it.

Recipe (the decoder activations of the xDiT LTX-2.5 pages are replaced by
N(0,1) draws of the same shapes; no model weights or dataset are involved):

1. one ``torch.Generator`` on the target device, seeded per workload;
2. ``q = bf16(randn * HD**-0.5)`` -- Q arrives pre-scaled by head_dim**-0.5
   (aiter PR page, Technical Details, public launcher paragraph);
3. ``k = randn``; for the full-scale workload every element is independently
   multiplied by 8 with probability 0.01 (softmax-range stress), then bf16;
4. ``v = bf16(randn)``.

The draws are deterministic for a given (seed, device type, torch version);
CPU and GPU streams differ, so a test generates once and copies the same
bytes to both sides.

RMSNorm inputs (the transformer block norms of the xDiT LTX-2.5 PR page,
Changes item 2; the pages give no hidden size or token count, so a stand-in
of 24576 tokens x 4096 channels is used): ``x = bf16(randn * exp(randn_row))``
-- N(0,1) channels with a log-normal per-token scale, since hidden-state
magnitudes vary from token to token -- and ``weight = bf16(1 + 0.1 * randn)``,
a norm weight near its ones initialisation.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    shape: tuple  # (B, T, H, W, NH, HD)
    window: tuple  # (KT, KH, KW)
    seed: int
    k_outlier_frac: float = 0.0
    k_outlier_scale: float = 8.0
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        B, T, H, W, _, _ = self.shape
        return B * T * H * W

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs: 4 * B*NH*T*H*W * KT*KH*KW * HD."""
        B, T, H, W, NH, HD = self.shape
        KT, KH, KW = self.window
        return 4 * B * NH * T * H * W * KT * KH * KW * HD

    @property
    def bytes(self) -> int:
        """Compulsory HBM bytes: q, k, v read once and out written once (bf16)."""
        B, T, H, W, NH, HD = self.shape
        return 4 * B * T * H * W * NH * HD * 2


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", (1, 4, 12, 16, 2, 32), (3, 5, 5), 0,
                 note="oracle finishes well under a second"),
        Workload("decoder_tile", (1, 16, 64, 96, 8, 64), (3, 7, 7), 1,
                 note="one VAE-decoder tile"),
        Workload("narrow_w7", (1, 16, 64, 7, 8, 64), (3, 5, 7), 2,
                 note="edge tile with W equal to KW"),
        Workload("narrow_w5", (1, 16, 64, 5, 8, 64), (3, 5, 5), 3,
                 note="edge tile with W equal to KW"),
        Workload("large_window", (1, 16, 48, 64, 8, 64), (11, 11, 11), 4,
                 note="1331 keys per query"),
        Workload("full_scale", (1, 32, 128, 192, 16, 128), (3, 7, 7), 5,
                 k_outlier_frac=0.01, k_outlier_scale=8.0,
                 note="1% of k elements x8"),
        Workload("wide_w27", (1, 4, 8, 128, 8, 64), (3, 5, 27), 6,
                 note="anisotropic wide window; grid of the aiter PR's (3,5,27) "
                      "benchmark row (its head count is not stated; 8 here)"),
        Workload("window_19", (1, 24, 32, 32, 4, 64), (19, 19, 19), 8,
                 note="a 484-key window union per 4x4 query block: the four-group "
                      "rolling instantiation"),
        Workload("window_19_hd128", (1, 24, 32, 32, 2, 128), (19, 19, 19), 9,
                 note="the same window at head dim 128, whose halo no rolling "
                      "instantiation's LDS holds: the general family's case"),
        Workload("wide_w41", (1, 4, 8, 128, 8, 64), (3, 5, 41), 7,
                 note="a window wider than 33 along W (the Triton kernel's shape gate "
                      "sent these to tiled SDPA) on the same grid"),
    )
}


@dataclass(frozen=True)
class NormWorkload:
    name: str
    rows: int
    dim: int
    seed: int
    note: str = field(default="", compare=False)

    @property
    def bytes(self) -> int:
        """Compulsory HBM bytes: x read once, y written once, the weight read once."""
        return 2 * self.rows * self.dim * 2 + self.dim * 2


NORM_WORKLOADS = {
    w.name: w
    for w in (
        NormWorkload("rms_tiny", 37, 520, 20, note="ragged: 65 16-byte pieces per row"),
        NormWorkload("rms_block_norm", 24576, 4096, 21,
                     note="stand-in for one block norm over a video latent: 24576 tokens "
                          "(16 x 32 x 48) x 4096 channels"),
    )
}


def make_norm_inputs(rows: int, dim: int, seed: int, device="cpu"):
    """Draw (x, weight): x (rows, dim) and weight (dim,), contiguous bf16."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    scale = torch.exp(torch.randn((rows, 1), generator=g, device=dev))
    x = (torch.randn((rows, dim), generator=g, device=dev) * scale).to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn((dim,), generator=g, device=dev)).to(torch.bfloat16)
    return x, w


def make_inputs(shape, seed: int, device="cpu", k_outlier_frac: float = 0.0,
                k_outlier_scale: float = 8.0):
    """Draw (q, k, v) as contiguous bf16 tensors of ``shape`` on ``device``."""
    shape = tuple(int(s) for s in shape)
    hd = shape[-1]
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    q = (torch.randn(shape, generator=g, device=dev) * (hd ** -0.5)).to(torch.bfloat16)
    k = torch.randn(shape, generator=g, device=dev)
    if k_outlier_frac > 0.0:
        hit = torch.rand(shape, generator=g, device=dev) < k_outlier_frac
        k = torch.where(hit, k * k_outlier_scale, k)
        del hit
    k = k.to(torch.bfloat16)
    v = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    return q, k, v


def make_spike_inputs(shape, seed: int, spikes, device="cpu"):
    """(q, k, v) whose scores hold a few extreme keys: q is ones/HD plus a
    little noise, k and v are standard normal, and for every (t, h, w, s) in
    ``spikes`` the key at that grid position (all batches and heads) is the
    constant s, so its score is about s (and s*(1 +- 0.25) across queries)
    against scores of about +-0.2 elsewhere."""
    shape = tuple(int(x) for x in shape)
    hd = shape[-1]
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    q = (1.0 / hd + torch.randn(shape, generator=g, device=dev) * (0.25 / hd ** 0.5)).to(torch.bfloat16)
    k = torch.randn(shape, generator=g, device=dev)
    for (t, h, w, s) in spikes:
        k[:, t, h, w] = float(s)
    k = k.to(torch.bfloat16)
    v = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    return q, k, v


def workload_inputs(name: str, device="cpu"):
    w = WORKLOADS[name]
    return make_inputs(w.shape, w.seed, device, w.k_outlier_frac, w.k_outlier_scale)


def sha256_of(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (recorded next to results)."""
    a = t.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    return hashlib.sha256(memoryview(a)).hexdigest()
