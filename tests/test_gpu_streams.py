"""GPU check that the composites keep no per-call state outside their
arguments: two gated MLPs (different shapes, scales and workspaces) and a
split-QKV call launched concurrently on two streams (default priority) give
bitwise what the same calls give one after another on one stream."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin

from gpu_util import device, scalar, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


def _mlp(seed, M, H, I, dev):
    wl = workloads.gated_mlp(seed, M, H, I)
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    q, s = {}, {}
    for k, w in wl.weights.items():
        q[k], s[k] = olin.rtn_weight(w)
    args = dict(x=to_dev_bf16(wl.x, dev), sx=scalar(sx, dev),
                wg=to_dev_u8(q["gate"], dev), sg=scalar(s["gate"], dev),
                wu=to_dev_u8(q["up"], dev), su=scalar(s["up"], dev),
                sh=scalar(np.float32(0.05), dev),
                wd=to_dev_u8(q["down"], dev), sd=scalar(s["down"], dev))
    ws = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    return args, ws, y


def _run_mlp(p):
    a, ws, y = p
    fp8.gated_mlp_fp8(a["x"], a["sx"], a["wg"], a["sg"], a["wu"], a["su"], a["sh"],
                      a["wd"], a["sd"], out=y, workspace=ws)


def _qkv(dev):
    wl = workloads.split_qkv(seed=3, M=1024, H=2048, N=2048)
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    ws, ss = [], []
    for k in ("q", "k", "v"):
        qw, sw = olin.rtn_weight(wl.weights[k])
        ws.append(to_dev_u8(qw, dev))
        ss.append(scalar(sw, dev))
    outs = tuple(torch.empty((1024, 2048), dtype=torch.bfloat16, device=dev) for _ in range(3))
    work = torch.empty(fp8.qkv_fp8_workspace(1024, 2048), dtype=torch.uint8, device=dev)
    return (to_dev_bf16(wl.x, dev), scalar(sx, dev), ws, ss, outs, work)


def _run_qkv(p):
    x, sx, ws, ss, outs, work = p
    fp8.qkv_fp8(x, sx, ws[0], ss[0], ws[1], ss[1], ws[2], ss[2], outs=outs, workspace=work)


def test_composites_on_two_streams_equal_sequential():
    dev = device()
    p1 = _mlp(11, 2048, 1024, 4096, dev)
    p2 = _mlp(12, 512, 2048, 6144, dev)
    pq = _qkv(dev)
    # one after another on the current stream
    _run_mlp(p1)
    _run_mlp(p2)
    _run_qkv(pq)
    torch.cuda.synchronize()
    ref = [p1[2].clone(), p2[2].clone()] + [t.clone() for t in pq[4]]
    for t in [p1[2], p2[2], *pq[4]]:
        t.fill_(0)
    torch.cuda.synchronize()
    # concurrently: the first MLP on one stream, the second MLP and the
    # split-QKV call on another, several times over
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    start = torch.cuda.Event()
    start.record(torch.cuda.current_stream(dev))
    s1.wait_event(start)
    s2.wait_event(start)
    for _ in range(3):
        with torch.cuda.stream(s1):
            _run_mlp(p1)
        with torch.cuda.stream(s2):
            _run_mlp(p2)
            _run_qkv(pq)
    torch.cuda.synchronize()
    got = [p1[2], p2[2], *pq[4]]
    for r, g in zip(ref, got):
        assert torch.equal(r.view(torch.int16), g.view(torch.int16))
