"""GPU: the fused-topology comparison -- re-quantization of a group onto its
largest scale (the failure mode the split path avoids) and GEMMs that write
column slices of one [M, 2N] buffer with the right row stride (pull request
"Load static FP8 Cosmos3 Nano/Super checkpoints without re-quantizing them",
"Description" and "What changed")."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin
from oracle.swiglu import silu_mul_adjacent_fp8, silu_mul_ab_f64

from oracle.formats import bf16_ulps, f32_to_bf16

from gpu_util import (check_fp8_tolerance, check_gemm_f32, device, host_bits,
                      host_f32, host_u8, scalar, to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ratio", [1.0, 0.5, 0.3, 1.0 / 7, 2.0 ** -9])
def test_requantize_all_codes_bitexact(ratio):
    # every code (NaNs included) at s_member = ratio * s_max
    dev = device()
    codes = np.tile(np.arange(256, dtype=np.uint8), 17)[:4097]   # ragged tail
    s_max = np.float32(0.0173)
    s_i = np.float32(np.float32(ratio) * s_max)
    want, _ = olin.requantize_onto_max([codes, codes], [s_i, s_max])
    group = torch.tensor([s_i, s_max], dtype=torch.float32, device=dev)
    got = host_u8(fp8.fp8_requantize_onto_max(to_dev_u8(codes, dev), scalar(s_i, dev), group))
    assert np.array_equal(got, want[0])
    if ratio == 1.0:
        nan = (codes & 0x7F) == 0x7F
        assert np.array_equal(got[~nan], codes[~nan])     # the max member is unchanged


def test_requantize_changes_the_smaller_members_codes():
    dev = device()
    rng = np.random.default_rng(61)
    w = workloads.to_bf16_bits(rng.standard_normal((256, 512)).astype(np.float32) * np.float32(0.02))
    q, s = olin.rtn_weight(w)
    s_big = np.float32(s * np.float32(1.37))
    group = torch.tensor([s, s_big], dtype=torch.float32, device=dev)
    got = host_u8(fp8.fp8_requantize_onto_max(to_dev_u8(q.ravel(), dev), scalar(s, dev), group))
    want, _ = olin.requantize_onto_max([q.ravel(), q.ravel()], [s, s_big])
    assert np.array_equal(got, want[0])
    assert np.mean(got != q.ravel()) > 0.3


@pytest.mark.parametrize("M,N,K", [(37, 64, 144), (300, 13, 64), (257, 384, 1040)])
def test_gemms_into_column_slices(M, N, K):
    # two projections into [:, 0:N) and [:, N:2N) of one [M, 2N + 3] buffer:
    # each slice equals its own fp8_linear bitwise and nothing else is written
    dev = device()
    rng = np.random.default_rng(M * 3 + N)
    qx = to_dev_u8(rng.integers(0, 0x7E, (M, K), dtype=np.uint8), dev)
    qa = to_dev_u8(rng.integers(0, 0x7E, (N, K), dtype=np.uint8), dev)
    qb = to_dev_u8(rng.integers(0, 0x7E, (N, K), dtype=np.uint8), dev)
    sx, sa, sb = scalar(0.01, dev), scalar(0.02, dev), scalar(0.03, dev)
    L = 2 * N + 3 if N % 4 else 2 * N + 8        # ragged (N = 13) and 16-byte rows
    buf = torch.full((M, L), -7.0, dtype=torch.bfloat16, device=dev)
    fp8.fp8_linear_into(qx, qa, sx, sa, buf, col0=0)
    if (N * 2) % 16 == 0:                        # the second slice must stay 16-byte aligned
        fp8.fp8_linear_into(qx, qb, sx, sb, buf, col0=N)
    ya = host_bits(fp8.fp8_linear(qx, qa, sx, sa))
    got = host_bits(buf)
    assert np.array_equal(got[:, :N], ya)
    if (N * 2) % 16 == 0:
        assert np.array_equal(got[:, N:2 * N], host_bits(fp8.fp8_linear(qx, qb, sx, sb)))
        rest = got[:, 2 * N:]
    else:
        rest = got[:, N:]
    assert np.all(rest == host_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0])


def test_fused_topology_chain_against_oracle():
    # fused gate/up topology: re-quantize both onto max(s), one [M, 2I] GEMM,
    # one-input SwiGLU -- against the oracle's same chain, and different from
    # the split path's codes
    dev = device()
    rng = np.random.default_rng(62)
    M, H, I = 96, 256, 384
    x = workloads.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    wg = workloads.to_bf16_bits(rng.standard_normal((I, H)).astype(np.float32) * np.float32(0.02))
    wu = workloads.to_bf16_bits(rng.standard_normal((I, H)).astype(np.float32) * np.float32(0.045))
    sxv = olin.scale_from_amax(olin.amax_f32(x))
    qx = olin.quant_static(x, sxv)
    qg, sg = olin.rtn_weight(wg)
    qu, su = olin.rtn_weight(wu)
    (rg, ru), smax = olin.requantize_onto_max([qg, qu], [sg, su])
    # oracle: [M, 2I] BF16 from the fused weight, then SwiGLU on the halves
    S, _ = olin.gemm_exact(qx, np.concatenate([rg, ru]))
    ybf = olin.epilogue_bf16(S, sxv, smax)
    h = silu_mul_ab_f64(ybf[:, :I], ybf[:, I:])
    sh = np.float32(np.max(np.abs(h)) / 448)
    # GPU: the same chain from the split codes
    group = torch.tensor([sg, su], dtype=torch.float32, device=dev)
    dg = fp8.fp8_requantize_onto_max(to_dev_u8(qg, dev), scalar(sg, dev), group)
    du = fp8.fp8_requantize_onto_max(to_dev_u8(qu, dev), scalar(su, dev), group)
    assert np.array_equal(host_u8(dg), rg) and np.array_equal(host_u8(du), ru)
    wf = torch.cat([dg, du])
    dqx = to_dev_u8(qx, dev)
    y = fp8.fp8_linear(dqx, wf, scalar(sxv, dev), scalar(smax, dev))
    y32 = host_f32(fp8.fp8_linear(dqx, wf, scalar(sxv, dev), scalar(smax, dev), out_kind=fp8.OUT_F32))
    S_full, A_full = olin.gemm_exact(qx, np.concatenate([rg, ru]))
    check_gemm_f32(y32, S_full, A_full, olin.epilogue_alpha(sxv, smax))
    yb = host_bits(y)
    assert np.array_equal(yb, f32_to_bf16(y32))
    # the oracle SwiGLU on the GPU's own [M, 2I] BF16 output
    q = host_u8(fp8.silu_mul_fp8(y, scalar(sh, dev)))
    check_fp8_tolerance(q.ravel(), silu_mul_adjacent_fp8(yb, sh).ravel())
    assert np.max(np.abs(bf16_ulps(yb, ybf))) <= 8
    # the split path keeps each member's own codes: the gate member changed
    assert np.mean(rg != qg) > 0.3
