"""The entry points allocate nothing, copy nothing between host and device
and never synchronise, so they can be captured in a HIP graph and replayed
(the xDiT LTX-2.5 RMSNorm change exists so that graph capture is not skipped
at the norm's call sites: xDiT PR 759 page, Changes item 2).  Every replay,
with eager work and synchronisation in between, must reproduce the eager
results bitwise and follow in-place changes of the inputs."""
import pytest
import torch

import neighborhood_attention_amd as na
from na3d_inputs import make_inputs, make_norm_inputs

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    ks = (3, 7, 7)
    q, k, v = make_inputs((1, 8, 32, 48, 2, 64), 400, "cuda")
    tiles = [make_inputs(d + (2, 64), 401 + i, "cuda")
             for i, d in enumerate([(1, 8, 32, 48), (1, 8, 32, 7)])]
    x, w = make_norm_inputs(300, 2048, 402, "cuda")
    out = torch.empty_like(q)
    y = torch.empty_like(x)
    touts = [torch.empty_like(t[0]) for t in tiles]

    def work():
        na.fwd(q, k, v, ks, out=out)
        na.rms_norm(x, w, 1e-6, out=y)
        na.fwd_batch(tiles, ks, outs=touts)

    # eager results, and a warm-up on a side stream before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (out.clone(), y.clone(), [t.clone() for t in touts])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(rep + 1.0)
        y.fill_(rep + 1.0)
        for t in touts:
            t.fill_(rep + 1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), rep
        assert torch.equal(y, ref[1]), rep
        assert all(torch.equal(a, b) for a, b in zip(touts, ref[2])), rep

    # the graph reads the inputs where they are: change them in place
    x.mul_(2.0)                      # RMSNorm is scale invariant (eps aside)
    q.copy_(q.flip(2))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    eager_out = na.fwd(q, k, v, ks)
    eager_y = na.rms_norm(x, w, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(out, eager_out)
    assert torch.equal(y, eager_y)
