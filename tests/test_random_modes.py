"""Randomised GPU parity over the supported contract: a fixed-seed draw of
small valid problems, each run through one entry point (contiguous,
strided views of a fused QKV buffer into a strided output, a query box with
windows in the whole grid, or a batch of independent grids) and compared with
the oracle on every output element."""
import random

import numpy as np
import pytest
import torch

import neighborhood_attention_amd as na
import oracle
from na3d_inputs import make_inputs

pytestmark = pytest.mark.gpu


def _check(got, ref, what):
    got = got.detach().cpu().double().numpy()
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    mab = float(np.abs(got - ref).max())
    assert np.isfinite(got).all() and rel <= 4e-3 and mab <= 5e-2, (what, rel, mab)


def _cases(seed, n):
    rng = random.Random(seed)
    for i in range(n):
        B = rng.choice([1, 1, 2])
        T, H, W = rng.randint(1, 12), rng.randint(1, 24), rng.randint(1, 40)
        NH = rng.randint(1, 3)
        HD = rng.choice([16, 32, 64, 64, 128, 256])
        ks = tuple(rng.randint(1, min(L, 13)) for L in (T, H, W))
        mode = rng.choice(["plain", "strided", "subgrid", "batch"])
        yield i, rng, mode, (B, T, H, W, NH, HD), ks


@pytest.mark.parametrize("case", list(range(60)))
def test_random_case(case):
    i, rng, mode, shape, ks = [c for c in _cases(2024 + case, 1)][0]
    B, T, H, W, NH, HD = shape
    print("case %d mode=%s shape=%s window=%s" % (case, mode, shape, ks), flush=True)
    if mode == "batch":
        tiles = []
        for j in range(rng.randint(1, 4)):
            d = (rng.choice([1, 2]), rng.randint(ks[0], max(ks[0], 10)),
                 rng.randint(ks[1], max(ks[1], 20)), rng.randint(ks[2], max(ks[2], 36)))
            tiles.append(make_inputs(d + (NH, HD), 3000 + 10 * case + j, "cuda"))
        outs = na.fwd_batch(tiles, ks)
        torch.cuda.synchronize()
        for (q, k, v), o in zip(tiles, outs):
            _check(o, oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks), "batch")
        return
    q, k, v = make_inputs(shape, 3000 + case, "cuda")
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), ks)
    if mode == "plain":
        out = na.fwd(q, k, v, ks)
    elif mode == "strided":
        qkv = torch.stack([q, k, v], dim=4).contiguous()      # (B,T,H,W,3,NH,HD)
        big = torch.zeros((B, T, H, W, NH + 1, HD), dtype=torch.bfloat16, device="cuda")
        out = big[:, :, :, :, :NH]
        na.fwd(qkv[:, :, :, :, 0], qkv[:, :, :, :, 1], qkv[:, :, :, :, 2], ks, out=out)
        torch.cuda.synchronize()
        assert torch.all(big[:, :, :, :, NH] == 0)             # the spare head is untouched
    else:
        t0, h0, w0 = rng.randint(0, T - 1), rng.randint(0, H - 1), rng.randint(0, W - 1)
        Tq, Hq, Wq = rng.randint(1, T - t0), rng.randint(1, H - h0), rng.randint(1, W - w0)
        out = na.fwd_subgrid(q[:, t0:t0 + Tq, h0:h0 + Hq, w0:w0 + Wq], k, v, ks, (t0, h0, w0))
        ref = ref[:, t0:t0 + Tq, h0:h0 + Hq, w0:w0 + Wq]
    torch.cuda.synchronize()
    _check(out, ref, mode)
