"""GPU: the fp8mot custom ops -- opcheck, torch.compile(fullgraph=True)
(dynamo + AOT autograd, eager backend: no generated kernels) and HIP graph
capture with replays checked against eager results."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
import mlp_fp8_quant_amd.torch_ops  # noqa: F401
from mlp_fp8_quant_amd import workloads

from gpu_util import device, scalar, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu
ops = torch.ops.fp8mot


def _mlp(dev, M=128, H=256, I=512, seed=71):
    rng = np.random.default_rng(seed)
    x = to_dev_bf16(workloads.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32)).ravel(), dev).view(M, H)
    w = lambda n, k: to_dev_u8(rng.integers(0, 0x7E, (n, k), dtype=np.uint8), dev)
    return dict(x=x, s=scalar(0.01, dev), sw=scalar(0.002, dev), sh=scalar(0.05, dev),
                wg=w(I, H), wu=w(I, H), wd=w(H, I))


def test_opcheck_every_op():
    dev = device()
    t = _mlp(dev)
    x, s, sw, sh = t["x"], t["s"], t["sw"], t["sh"]
    q = ops.quant_static(x, s)
    y = ops.linear(q, t["wg"], s, sw)
    qr, sr = ops.quant_per_row(x)
    y2 = torch.cat([y, y], dim=-1).contiguous()
    cases = [
        (ops.quant_static, (x, s)),
        (ops.linear, (q, t["wg"], s, sw)),
        (ops.silu_mul_2in, (y, y, sh, 1.702, 1.0)),
        (ops.silu_mul, (y2, sh)),
        (ops.gated_mlp, (x, s, t["wg"], sw, t["wu"], sw, sh, t["wd"], sw)),
        (ops.qkv, (x, s, t["wg"], sw, t["wu"], sw, t["wg"], sw)),
        (ops.quant_per_row, (x,)),
        (ops.linear_rowwise, (qr, t["wg"], sr, torch.full((512,), 0.002, device=dev))),
    ]
    for op, args in cases:
        torch.library.opcheck(op, args, test_utils=("test_schema", "test_faketensor",
                                                     "test_aot_dispatch_dynamic"))


def test_compile_fullgraph_matches_eager():
    dev = device()
    t = _mlp(dev)

    def block(x):
        yq, yk, yv = ops.qkv(x, t["s"], t["wg"], t["sw"], t["wu"], t["sw"], t["wg"], t["sw"])
        h = ops.gated_mlp(x, t["s"], t["wg"], t["sw"], t["wu"], t["sw"], t["sh"], t["wd"], t["sw"])
        return h, yq

    compiled = torch.compile(block, fullgraph=True, backend="aot_eager")
    a = block(t["x"])
    b = compiled(t["x"])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_hip_graph_capture_replays_match_eager():
    # capture the gated MLP and the split QKV; replay several times with eager
    # work and synchronizations between the replays, every replay checked
    dev = device()
    t = _mlp(dev)
    x_static = t["x"].clone()

    def run():
        h = ops.gated_mlp(x_static, t["s"], t["wg"], t["sw"], t["wu"], t["sw"], t["sh"],
                          t["wd"], t["sw"])
        yq, yk, yv = ops.qkv(x_static, t["s"], t["wg"], t["sw"], t["wu"], t["sw"],
                             t["wg"], t["sw"])
        return h, yv

    want_h, want_v = run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            run()                          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_h, out_v = run()
    for r in range(4):
        noise = torch.randn_like(x_static.float())   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_h, want_h), f"replay {r}: gated MLP differs"
        assert torch.equal(out_v, want_v), f"replay {r}: qkv differs"
        del noise
    # new input values copied into the captured input buffer change the output
    x_static.copy_(t["x"] * 0.5)
    g.replay()
    torch.cuda.synchronize()
    assert not torch.equal(out_h, want_h)
