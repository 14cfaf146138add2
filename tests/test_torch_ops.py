"""The torch.library registrations (neighborhood_attention_amd.torch_ops):
the ops exist, trace as single opaque functional nodes with fake tensors (no
GPU needed), and on the GPU match the plain binding bitwise, pass
torch.library's schema and fake-tensor checks, and compile without graph
breaks."""
import pytest
import torch
from torch.fx.experimental.proxy_tensor import make_fx

import neighborhood_attention_amd as na
import neighborhood_attention_amd.torch_ops as ops


def test_ops_registered_without_mutation():
    for op in (torch.ops.na3d_amd.rms_norm.default, torch.ops.na3d_amd.na3d_fwd.default):
        schema = op._schema
        assert not any(a.alias_info is not None and a.alias_info.is_write for a in schema.arguments)


def test_trace_is_one_functional_node():
    def f(x, w):
        return ops.rms_norm(x, w, 1e-6) * 2

    x = torch.empty(3, 4096, dtype=torch.bfloat16, device="meta")
    w = torch.empty(4096, dtype=torch.bfloat16, device="meta")
    gm = make_fx(f, tracing_mode="fake")(x, w)
    targets = [n.target for n in gm.graph.nodes if n.op == "call_function"]
    assert torch.ops.na3d_amd.rms_norm.default in targets
    q = torch.empty(1, 4, 8, 8, 2, 64, dtype=torch.bfloat16, device="meta")
    gm = make_fx(lambda a: ops.na3d_fwd(a, a, a, [3, 5, 5]), tracing_mode="fake")(q)
    node = [n for n in gm.graph.nodes if n.target == torch.ops.na3d_amd.na3d_fwd.default][0]
    assert tuple(node.meta["val"].shape) == tuple(q.shape)


def test_module_parameters():
    m = ops.RMSNorm(256, eps=1e-5)
    assert m.weight.shape == (256,) and m.weight.dtype == torch.bfloat16
    assert not m.weight.requires_grad
    assert ops.RMSNorm(256, elementwise_affine=False).weight is None


@pytest.mark.gpu
def test_ops_on_gpu():
    from na3d_inputs import make_inputs, make_norm_inputs

    x, w = make_norm_inputs(96, 1024, 500, "cuda")
    x3 = x.view(4, 24, 1024)
    y = torch.ops.na3d_amd.rms_norm(x3, w, 1e-6)
    assert torch.equal(y.view(96, 1024), na.rms_norm(x, w, 1e-6))
    m = ops.RMSNorm(1024, eps=1e-6, device="cuda")
    with torch.no_grad():
        m.weight.copy_(w)
    assert torch.equal(m(x3), y)
    assert torch.equal(ops.RMSNorm(1024, elementwise_affine=False).cuda()(x), na.rms_norm(x, None))
    q, k, v = make_inputs((1, 4, 8, 8, 2, 64), 501, "cuda")
    assert torch.equal(torch.ops.na3d_amd.na3d_fwd(q, k, v, [3, 5, 5]), na.fwd(q, k, v, (3, 5, 5)))
    for op, args in ((torch.ops.na3d_amd.rms_norm.default, (x3, w, 1e-6)),
                     (torch.ops.na3d_amd.na3d_fwd.default, (q, k, v, [3, 5, 5]))):
        torch.library.opcheck(op, args, test_utils=("test_schema", "test_faketensor"))
    f = torch.compile(lambda a, b: ops.rms_norm(a, b, 1e-6), backend="eager", fullgraph=True)
    assert torch.equal(f(x3, w), y)
    torch.cuda.synchronize()
