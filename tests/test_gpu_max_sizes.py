"""GPU parity at the largest sizes the C ABI accepts.

The GEMM kernels address one tile's 256 operand rows of K codes and its 256
output rows with 32-bit byte offsets, so the library refuses K, N or ldc
beyond those windows (the refusals are checked on the CPU in
test_boundary_cpu.py).  Here the largest accepted K and the largest accepted
BF16 / FP32 output rows run on the GPU against the oracle, and the static
quantize runs over more than 2^31 elements (64-bit element indexing, ragged
tail) checked bit for bit everywhere."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from oracle import linear as olin
from oracle.formats import bf16_ulps, f32_to_bf16

from gpu_util import (check_gemm_bf16, check_gemm_f32, check_gemm_fp8_engine,
                      device, fp8_mfma_group_bound, host_bits, host_f32, scalar,
                      to_dev_u8)

pytestmark = pytest.mark.gpu

K_MAX = 8388576                    # largest K (multiple of 16) with 256 * K < 0x7FFFF000
N_MAX_BF16 = 0x7FFFF000 // 512 - 1
N_MAX_F32 = 0x7FFFF000 // 1024 - 1


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_gemm_largest_k(accum):
    # [300, K_MAX] x [200, K_MAX]: zeros except 40 blocks of 16 consecutive,
    # 16-aligned K positions (the first, the last and 38 spread between), so
    # the oracle's exact sum over those columns is the whole sum and the FP8
    # engine's 8-product groups are unchanged by the compaction
    dev = device()
    M, N, K = 300, 200, K_MAX
    rng = np.random.default_rng(77)
    blocks = np.unique(np.concatenate([[0, K // 16 - 1],
                                       rng.choice(K // 16, 38, replace=False)]))
    cols = (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
    sa, sb = _codes(rng, (M, cols.size)), _codes(rng, (N, cols.size))
    qa = torch.zeros((M, K), dtype=torch.uint8, device=dev)
    qb = torch.zeros((N, K), dtype=torch.uint8, device=dev)
    idx = torch.from_numpy(cols).to(dev)
    qa[:, idx] = to_dev_u8(sa, dev)
    qb[:, idx] = to_dev_u8(sb, dev)
    sx, sw = np.float32(0.0213), np.float32(1.7e-4)
    y32 = fp8.fp8_linear(qa, qb, scalar(sx, dev), scalar(sw, dev), fp8.OUT_F32, accum=accum)
    yb = fp8.fp8_linear(qa, qb, scalar(sx, dev), scalar(sw, dev), fp8.OUT_BF16, accum=accum)
    torch.cuda.synchronize()
    del qa, qb
    S, A = olin.gemm_exact(sa, sb)
    alpha = olin.epilogue_alpha(sx, sw)
    f = host_f32(y32)
    if accum == fp8.ACC_EXACT:
        check_gemm_f32(f, S, A, alpha)
        check_gemm_bf16(host_bits(yb), f, S, A, alpha)
    else:
        check_gemm_fp8_engine(f, S, A, alpha, fp8_mfma_group_bound(sa, sb))
    assert np.array_equal(host_bits(yb), f32_to_bf16(f))


@pytest.mark.parametrize("out_kind,N", [(fp8.OUT_BF16, N_MAX_BF16), (fp8.OUT_F32, N_MAX_F32)])
def test_gemm_widest_output_rows(out_kind, N):
    # the widest accepted output rows (N is odd: the BF16 epilogue takes its
    # per-element store path), every output against the oracle
    dev = device()
    M, K = 5, 32
    rng = np.random.default_rng(N)
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx, sw = np.float32(0.031), np.float32(2.5e-3)
    da, dsx, dsw = to_dev_u8(qa, dev), scalar(sx, dev), scalar(sw, dev)
    y = fp8.fp8_linear(da, to_dev_u8(qb, dev), dsx, dsw, out_kind)
    torch.cuda.synchronize()
    S, A = olin.gemm_exact(qa, qb)
    alpha = olin.epilogue_alpha(sx, sw)
    if out_kind == fp8.OUT_F32:
        check_gemm_f32(host_f32(y), S, A, alpha)
        return
    # BF16 rows this wide have no FP32 twin (its rows would exceed the
    # window); outputs beyond 1 ulp of the oracle's rounding (near
    # cancellation) get their FP32 values from a launch over just those
    # weight rows -- K = 32 is one stage, so every output sums in the same
    # order at any N
    yb = host_bits(y)
    ref = f32_to_bf16((S.astype(np.float32) * np.float32(alpha)).astype(np.float32))
    far = np.unique(np.nonzero(bf16_ulps(yb, ref) > 1)[1])
    if far.size:
        f = host_f32(fp8.fp8_linear(da, to_dev_u8(qb[far], dev), dsx, dsw, fp8.OUT_F32))
        check_gemm_bf16(yb[:, far], f, S[:, far], A[:, far], alpha)


def test_quant_static_beyond_2_to_31_elements():
    # x cycles through all 65,536 BF16 bit patterns for 2^31 + 40 elements
    # (a ragged tail of 8 past the last 16-element unit); every code must be
    # the oracle's code of its pattern
    dev = device()
    n = (1 << 31) + 40
    s = np.float32(0.0173)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    table = olin.quant_static(pats, s)
    reps = n // 65536 + 1
    x = torch.from_numpy(pats.view(np.int16)).to(dev).repeat(reps)[:n].view(torch.bfloat16)
    q = fp8.fp8_quant_static(x, scalar(s, dev))
    want = to_dev_u8(table, dev).repeat(reps)[:n]
    torch.cuda.synchronize()
    assert torch.equal(q, want)
