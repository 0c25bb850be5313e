"""Custom-op contract on the CPU: every fp8mot op has a fake kernel with the
right output shapes and dtypes, and a function of the ops traces into one
graph with fake tensors -- without running the library (pull request "Load
static FP8 Cosmos3 Nano/Super checkpoints without re-quantizing them", first
commit message: register_fake / opcheck / fullgraph)."""

import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

import mlp_fp8_quant_amd.torch_ops  # noqa: F401  (registers torch.ops.fp8mot)

ops = torch.ops.fp8mot


def _inputs(mode):
    with mode:
        d = "cuda"
        x = torch.empty((2, 48, 256), dtype=torch.bfloat16, device=d)
        s = torch.empty(1, dtype=torch.float32, device=d)
        wg = torch.empty((512, 256), dtype=torch.uint8, device=d)
        wd = torch.empty((256, 512), dtype=torch.uint8, device=d)
        return x, s, wg, wd


def test_fake_kernels_shapes_and_dtypes():
    mode = FakeTensorMode()
    x, s, wg, wd = _inputs(mode)
    with mode:
        q = ops.quant_static(x, s)
        assert q.shape == x.shape and q.dtype == torch.uint8
        y = ops.linear(q, wg, s, s)
        assert y.shape == (2, 48, 512) and y.dtype == torch.bfloat16
        h = ops.silu_mul_2in(y, y, s, 1.702, 1.0)
        assert h.shape == y.shape and h.dtype == torch.uint8
        h1 = ops.silu_mul(y, s)
        assert h1.shape == (2, 48, 256) and h1.dtype == torch.uint8
        o = ops.gated_mlp(x, s, wg, s, wg, s, s, wd, s)
        assert o.shape == x.shape and o.dtype == torch.bfloat16
        yq, yk, yv = ops.qkv(x, s, wg, s, wd, s, wd, s)
        assert yq.shape == (2, 48, 512) and yk.shape == (2, 48, 256) and yv.dtype == torch.bfloat16
        qr, sr = ops.quant_per_row(x)
        assert qr.shape == x.shape and sr.shape == (2, 48) and sr.dtype == torch.float32
        yr = ops.linear_rowwise(qr, wg, sr, sr)
        assert yr.shape == (2, 48, 512) and yr.dtype == torch.bfloat16


def test_gated_mlp_and_qkv_trace_into_one_graph():
    def block(x, s, wg, wd):
        yq, yk, yv = ops.qkv(x, s, wg, s, wg, s, wg, s)
        return ops.gated_mlp(x, s, wg, s, wg, s, s, wd, s), yq

    mode = FakeTensorMode()
    args = _inputs(mode)
    gm = make_fx(block, tracing_mode="fake")(*args)
    names = [str(n.target) for n in gm.graph.nodes if n.op == "call_function"]
    assert "fp8mot.qkv.default" in names and "fp8mot.gated_mlp.default" in names
