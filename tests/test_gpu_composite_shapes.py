"""GPU check of the composites' tile scheduling on assorted ragged shapes: the
fused gate/up + SwiGLU kernel (from a single tile to several per workgroup
in its persistent loop, ragged M and I, K = H a multiple of 128 or not)
bitwise equal to two fp8_linear calls + silu_mul_2in_fp8 when I >= H; and
the grouped split-Q/K/V launch (unequal member widths, an empty member)
bitwise equal to three fp8_linear calls on the one quantized activation."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads

from gpu_util import device, scalar, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu

# (M, I, H) with I >= H, ragged, from well under one tile per CU to several
FUSED = [(1, 48, 32), (77, 400, 160), (300, 1040, 1024), (1025, 2064, 1040), (2500, 3008, 1536),
         (4133, 4208, 2048), (6000, 5136, 4096)]
# (M, H, Nq, Nk, Nv)
QKV = [(64, 256, 256, 64, 64), (300, 1024, 1024, 256, 0), (1500, 2048, 2048, 512, 512),
       (3000, 4096, 4096, 1024, 1024), (2048, 1040, 3000, 16, 3000)]


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("M,I,H", FUSED)
def test_fused_gate_up_shapes_equal_parts(accum, M, I, H):
    dev = device()
    print(f"fused M={M} I={I} H={H} accum={accum}", flush=True)
    rng = np.random.default_rng(M * 31 + I * 7 + H + accum)
    qx, wg, wu = (to_dev_u8(_codes(rng, s), dev) for s in ((M, H), (I, H), (I, H)))
    dsx, dsg, dsu, dsh = (scalar(v, dev) for v in (0.02, 1e-3, 2e-3, 0.5))
    qh = fp8.fp8_gate_up_swiglu(qx, wg, dsx, dsg, wu, dsu, dsh, accum=accum)
    G = fp8.fp8_linear(qx, wg, dsx, dsg, accum=accum)
    U = fp8.fp8_linear(qx, wu, dsx, dsu, accum=accum)
    assert torch.equal(qh, fp8.silu_mul_2in_fp8(G, U, dsh))


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("M,H,Nq,Nk,Nv", QKV)
def test_qkv_grouped_shapes_equal_separate(accum, M, H, Nq, Nk, Nv):
    dev = device()
    print(f"qkv M={M} H={H} N={Nq},{Nk},{Nv} accum={accum}", flush=True)
    rng = np.random.default_rng(M + H + Nq + 3 * Nk + 7 * Nv + accum)
    x = to_dev_bf16(workloads.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32)), dev)
    sx = scalar(0.01, dev)
    ws = [to_dev_u8(_codes(rng, (n, H)), dev) for n in (Nq, Nk, Nv)]
    ss = [scalar(1e-3 * (i + 1), dev) for i in range(3)]
    yq, yk, yv = fp8.qkv_fp8(x, sx, ws[0], ss[0], ws[1], ss[1], ws[2], ss[2], accum=accum)
    qx = fp8.fp8_quant_static(x, sx)
    for y, w, s in zip((yq, yk, yv), ws, ss):
        assert y.shape == (M, w.shape[0])
        if w.shape[0]:
            assert torch.equal(y.view(torch.int16),
                               fp8.fp8_linear(qx, w, sx, s, accum=accum).view(torch.int16))
