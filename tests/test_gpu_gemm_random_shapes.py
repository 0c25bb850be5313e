"""GPU parity of fp8_linear (exact engine) on seeded random shapes that reach
every tile configuration the library's shape rule picks, against the oracle's
exact sum: ragged M, N and K (K a multiple of 128 or not), the FP32 output on
every row (or, from 2048 rows on, on 64 rows that include the last 16) within
1e-5 * sum|terms|, and the BF16 output of the whole launch equal to the RNE of
its FP32 output.

The shapes were drawn from four size regimes with a fixed seed; the tile
configuration each takes (on 256 CUs) is noted beside it: 128x64 tiles with
and without the two-group K split, 128x128 with and without it, 256x128,
256x256 and 192x256."""

import numpy as np
import pytest

import mlp_fp8_quant_amd as fp8
from oracle import linear as olin
from oracle.formats import f32_to_bf16

from gpu_util import (check_gemm_bf16, check_gemm_f32, device, host_bits, host_f32,
                      report, scalar, to_dev_u8)

pytestmark = pytest.mark.gpu

SHAPES = [
    (49, 203, 96),       # 128x64
    (43, 95, 320),       # 128x64, K split
    (181, 240, 928),     # 128x64, K split
    (199, 24, 144),      # 128x64, K split
    (620, 249, 688),     # 128x64, K split
    (208, 1836, 1472),   # 128x64
    (258, 422, 1872),    # 128x64, K split
    (453, 1620, 2528),   # 128x64, K split
    (1486, 2421, 992),   # 128x128
    (1065, 4750, 16),    # 256x128
    (702, 3860, 144),    # 128x128
    (1475, 4566, 1632),  # 256x128
    (3288, 6984, 528),   # 192x256
    (2813, 4647, 320),   # 256x256
    (3916, 6213, 1264),  # 256x256
    (2695, 7604, 1344),  # 192x256
    (1800, 1700, 2064),  # 128x128, K split
    (2200, 5000, 1024),  # 192x256, K a multiple of 128
    (1000, 3000, 512),   # 128x128, K a multiple of 128
]


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_shape_against_oracle(M, N, K):
    dev = device()
    print(f"case M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = np.float32(rng.uniform(1e-3, 1e-1))
    sw = np.float32(rng.uniform(1e-4, 1e-2))
    da, db = to_dev_u8(qa, dev), to_dev_u8(qb, dev)
    dsx, dsw = scalar(sx, dev), scalar(sw, dev)
    y32 = host_f32(fp8.fp8_linear(da, db, dsx, dsw, fp8.OUT_F32))
    yb = host_bits(fp8.fp8_linear(da, db, dsx, dsw, fp8.OUT_BF16))
    assert np.array_equal(yb, f32_to_bf16(y32))       # one kernel, one sum
    if M < 2048:
        rows = np.arange(M)
    else:
        rows = np.concatenate([np.sort(rng.choice(M - 16, 48, replace=False)), np.arange(M - 16, M)])
    S, A = olin.gemm_exact(qa[rows], qb)
    alpha = olin.epilogue_alpha(sx, sw)
    check_gemm_f32(y32[rows], S, A, alpha)
    n2 = check_gemm_bf16(yb[rows], y32[rows], S, A, alpha)
    if n2:
        report(f"random_shape_{M}x{N}x{K}_r13_second_clause", n2)
