"""GPU check of gated_mlp_fp8_noalloc, the gated MLP for callers that cannot
allocate: through the C ABI it must give bit for bit what gated_mlp_fp8 with
a caller workspace gives, on consecutive calls of decreasing size (the
library's scratch keeps the previous call's qX and qH, which must not leak
into a smaller call), the first at the scratch's full 64 MiB, and under HIP
graph capture, the use it exists for."""

import pytest
import torch

import mlp_fp8_quant_amd as fp8

from gpu_util import device

pytestmark = pytest.mark.gpu


def _case(dev, gen, M, H, I):
    x = (torch.randn((M, H), device=dev, generator=gen) * 2.0).to(torch.bfloat16)
    w = {}
    s = {}
    for k, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w[k], s[k] = fp8.rtn_weight((torch.randn(shape, device=dev, generator=gen) * 0.02)
                                    .to(torch.bfloat16))
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st)
    sh = torch.tensor([0.004], dtype=torch.float32, device=dev)
    return x, w, s, sx, sh


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_noalloc_equals_workspace_entry_on_shrinking_calls(accum):
    dev = device()
    gen = torch.Generator(device=dev)
    gen.manual_seed(17 + accum)
    # 4096 x (4096 + 12288) codes fill the 64 MiB scratch exactly
    shapes = [(4096, 4096, 12288), (2048, 2048, 8192), (300, 512, 1040)]
    for M, H, I in shapes:
        print(f"gated_mlp_fp8_noalloc M={M} H={H} I={I} accum={accum}", flush=True)
        x, w, s, sx, sh = _case(dev, gen, M, H, I)
        args = (x, sx, w["gate"], s["gate"], w["up"], s["up"], sh, w["down"], s["down"])
        y_ws = fp8.gated_mlp_fp8(*args, accum=accum)
        y_na = torch.full_like(y_ws, 7.0)
        fp8.gated_mlp_fp8_noalloc(*args, out=y_na, accum=accum)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), (M, H, I)


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_noalloc_under_hip_graph_capture(accum):
    # the use the entry point is for: captured once in a HIP graph (no
    # allocation during capture), replayed with eager work and
    # synchronizations between replays, every replay bitwise the eager
    # workspace entry point's output; new input values copied into the
    # captured input change the replayed output to the eager output for them
    dev = device()
    gen = torch.Generator(device=dev)
    gen.manual_seed(29 + accum)
    M, H, I = 512, 1024, 2048
    x, w, s, sx, sh = _case(dev, gen, M, H, I)
    args = lambda xx: (xx, sx, w["gate"], s["gate"], w["up"], s["up"], sh,   # noqa: E731
                       w["down"], s["down"])
    want = fp8.gated_mlp_fp8(*args(x), accum=accum)
    x_in = x.clone()
    y = torch.empty_like(want)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(2):
            fp8.gated_mlp_fp8_noalloc(*args(x_in), out=y, accum=accum)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8.gated_mlp_fp8_noalloc(*args(x_in), out=y, accum=accum)
    for r in range(3):
        noise = torch.randn((1 << 20,), device=dev, generator=gen)   # eager work between replays
        y.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"replay {r}"
        del noise
    x2 = (x.float() * 0.5).to(torch.bfloat16)
    want2 = fp8.gated_mlp_fp8(*args(x2), accum=accum)
    x_in.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), want2.view(torch.int16))
    assert not torch.equal(want2.view(torch.int16), want.view(torch.int16))
    del g


def test_noalloc_refuses_sizes_beyond_its_scratch():
    dev = device()
    M, H, I = 4097, 4096, 12288
    x = torch.zeros((M, H), dtype=torch.bfloat16, device=dev)
    wg = torch.zeros((I, H), dtype=torch.uint8, device=dev)
    wd = torch.zeros((H, I), dtype=torch.uint8, device=dev)
    s = torch.ones(1, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    with pytest.raises(fp8.Fp8motError) as e:
        fp8.gated_mlp_fp8_noalloc(x, s, wg, s, wg, s, s, wd, s, out=y)
    assert e.value.status == 7
