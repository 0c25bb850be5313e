"""GPU parity: per-row FP8 -- per-token activation quantization, per-channel
weight RTN and the GEMM with a scale per row of each operand (model card
"Cosmos3-Nano-Policy-DROID, FP8 + RTN + moving-average activation observer",
section 3.2)."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle.formats import bf16_ulps, f32_to_bf16
from oracle.linear import gemm_exact
from oracle.rowwise import (epilogue_rowwise_alpha, epilogue_rowwise_f32,
                            quant_per_row)

from gpu_util import (check_gemm_fp8_engine, device, fp8_mfma_group_bound,
                      host_bits, host_f32, host_u8, to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu


def _rows(rng, rows, K, lo=1e-3, hi=1e3):
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x *= rng.uniform(lo, hi, (rows, 1)).astype(np.float32)
    return workloads.to_bf16_bits(x)


def _quant_dev(x, dev):
    q, s = fp8.fp8_quant_per_row(to_dev_bf16(x.ravel(), dev).view(x.shape))
    return host_u8(q), host_f32(s)


@pytest.mark.parametrize("rows,K", [(1, 16), (17, 2048), (33, 4096), (300, 5120), (7, 6160),
                                    (9, 8192), (64, 25600), (3, 48), (5, 32784)])
def test_quant_per_row_bitexact(rows, K):
    dev = device()
    x = _rows(np.random.default_rng(rows * 7 + K), rows, K)
    q, s = _quant_dev(x, dev)
    wq, ws = quant_per_row(x)
    assert np.array_equal(s.view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(q, wq)


def test_quant_per_row_special_rows_and_rank3():
    dev = device()
    rows = np.zeros((6, 32), np.float32)
    rows[1] = np.linspace(-3, 3, 32)
    rows[1, 5] = np.nan
    rows[2] = np.linspace(-1, 1, 32)
    rows[2, 7] = np.inf
    rows[3] = np.linspace(-448, 448, 32)
    rows[4] = 1e-30                    # tiny: its own scale brings it to 448
    rows[5, ::2] = -0.0
    x = workloads.to_bf16_bits(rows)
    x[0, 1::2] = 0x8000                # -0 in the zero row
    q, s = _quant_dev(x, dev)
    wq, ws = quant_per_row(x)
    assert np.array_equal(q, wq)
    assert np.array_equal(np.isnan(s), np.isnan(ws)) and np.array_equal(s[~np.isnan(s)], ws[~np.isnan(ws)])
    assert s[0] == 0 and s[5] == 0 and q[0, 1] == 0x80
    # rank 3: [2, 3, K] quantizes as 6 rows
    x3 = _rows(np.random.default_rng(5), 6, 64).reshape(2, 3, 64)
    q3, s3 = fp8.fp8_quant_per_row(to_dev_bf16(x3.ravel(), dev).view(2, 3, 64))
    assert q3.shape == (2, 3, 64) and s3.shape == (2, 3)
    wq3, ws3 = quant_per_row(x3.reshape(6, 64))
    assert np.array_equal(host_u8(q3).reshape(6, 64), wq3)
    assert np.array_equal(host_f32(s3).ravel(), ws3)


def _check_rowwise_f32(y32, S, A, alpha):
    a = alpha.astype(np.float64)
    err = np.abs(y32.astype(np.float64) - a * S)
    bad = err > 1e-5 * a * A
    assert not bad.any(), f"{bad.sum()} outputs exceed 1e-5*sum|terms|"


def _check_rowwise_bf16(yb, y32, S, A, alpha):
    ref32 = (S.astype(np.float32) * alpha).astype(np.float32)
    d = bf16_ulps(yb, f32_to_bf16(ref32))
    idx = d > 1
    if idx.any():   # the FP32 output passes 1e-5 and the BF16 output is its RNE
        a = alpha.astype(np.float64)
        ok32 = np.abs(y32[idx].astype(np.float64) - a[idx] * S[idx]) <= 1e-5 * a[idx] * A[idx]
        assert (ok32 & (f32_to_bf16(y32[idx]) == yb[idx])).all()


@pytest.mark.parametrize("engine", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_linear_rowwise_192_row_tiles_sampled_rows(engine):
    # 3000 x 6000 x 1024 takes 192x256 tiles (three 32-row blocks per wave,
    # ragged last tile row and column): the per-row epilogue on sampled rows,
    # the last ones included, against the oracle
    dev = device()
    M, N, K = 3000, 6000, 1024
    rng = np.random.default_rng(5 + engine)
    x = _rows(rng, M, K, 0.05, 20)
    w = _rows(rng, N, K, 0.002, 0.05)
    qx_d, sx_d = fp8.fp8_quant_per_row(to_dev_bf16(x.ravel(), dev).view(M, K))
    qw_d, sw_d = fp8.fp8_quant_per_row(to_dev_bf16(w.ravel(), dev).view(N, K))
    qw, sw = quant_per_row(w)
    assert np.array_equal(host_u8(qw_d), qw)
    rows = np.concatenate([np.arange(M - 40, M), np.sort(rng.choice(M - 40, 24, replace=False))])
    qx, sx = quant_per_row(x[rows])
    assert np.array_equal(host_u8(qx_d)[rows], qx)
    S, A = gemm_exact(qx, qw)
    alpha = epilogue_rowwise_alpha(sx, sw)
    y32 = host_f32(fp8.fp8_linear_rowwise(qx_d, qw_d, sx_d, sw_d, out_kind=fp8.OUT_F32, accum=engine))[rows]
    yb = host_bits(fp8.fp8_linear_rowwise(qx_d, qw_d, sx_d, sw_d, accum=engine))[rows]
    if engine == fp8.ACC_EXACT:
        _check_rowwise_f32(y32, S, A, alpha)
        _check_rowwise_bf16(yb, y32, S, A, alpha)
    else:
        check_gemm_fp8_engine(y32[:8], S[:8], A[:8], alpha[:8], fp8_mfma_group_bound(qx[:8], qw))
        assert np.array_equal(yb, f32_to_bf16(y32))


@pytest.mark.parametrize("engine", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (37, 129, 144), (300, 200, 4096), (257, 385, 1040), (5, 16, 0)])
def test_linear_rowwise_against_oracle(engine, M, N, K):
    dev = device()
    rng = np.random.default_rng(M + N + K + engine)
    x = _rows(rng, M, K, 0.05, 20)
    w = _rows(rng, N, K, 0.002, 0.05)
    qx_d, sx_d = fp8.fp8_quant_per_row(to_dev_bf16(x.ravel(), dev).view(M, K))
    qw_d, sw_d = fp8.fp8_quant_per_row(to_dev_bf16(w.ravel(), dev).view(N, K))
    qx, sx = quant_per_row(x)
    qw, sw = quant_per_row(w)
    assert np.array_equal(host_u8(qx_d), qx) and np.array_equal(host_u8(qw_d), qw)
    S, A = gemm_exact(qx, qw)
    alpha = epilogue_rowwise_alpha(sx, sw)
    y32 = host_f32(fp8.fp8_linear_rowwise(qx_d, qw_d, sx_d, sw_d, out_kind=fp8.OUT_F32, accum=engine))
    yb = host_bits(fp8.fp8_linear_rowwise(qx_d, qw_d, sx_d, sw_d, accum=engine))
    if engine == fp8.ACC_EXACT:
        _check_rowwise_f32(y32, S, A, alpha)
        _check_rowwise_bf16(yb, y32, S, A, alpha)
    else:
        check_gemm_fp8_engine(y32, S, A, alpha, fp8_mfma_group_bound(qx, qw))
        assert np.array_equal(yb, f32_to_bf16(y32))


def test_linear_rowwise_gen_mlp_shape_sampled_rows():
    # gate projection of the gen-tower MLP: M = 2048 tokens, N = 8192, K = 2048
    dev = device()
    rng = np.random.default_rng(77)
    M, N, K = 2048, 8192, 2048
    x = _rows(rng, M, K, 0.1, 10)
    w = workloads.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    qx_d, sx_d = fp8.fp8_quant_per_row(to_dev_bf16(x.ravel(), dev).view(M, K))
    qw_d, sw_d = fp8.fp8_quant_per_row(to_dev_bf16(w.ravel(), dev).view(N, K))
    y32 = host_f32(fp8.fp8_linear_rowwise(qx_d, qw_d, sx_d, sw_d, out_kind=fp8.OUT_F32))
    rows = np.sort(rng.choice(M, 48, replace=False))
    qx, sx = quant_per_row(x[rows])
    qw, sw = quant_per_row(w)
    assert np.array_equal(host_u8(qx_d)[rows], qx)
    S, A = gemm_exact(qx, qw)
    _check_rowwise_f32(y32[rows], S, A, epilogue_rowwise_alpha(sx, sw))


def test_quant_per_row_empty_rows_get_scale_zero():
    # K = 0: every row is empty, which the oracle scales as a zero row (0);
    # the scales start as NaN so a missing write shows
    dev = device()
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=dev)
    scales = torch.full((5,), float("nan"), dtype=torch.float32, device=dev)
    q, s = fp8.fp8_quant_per_row(x, scales=scales)
    wq, ws = quant_per_row(np.zeros((5, 0), np.uint16))
    assert q.shape == (5, 0) and np.array_equal(host_f32(s).view(np.uint32), ws.view(np.uint32))


def test_rowwise_refusals():
    dev = device()
    q = torch.zeros((4, 32), dtype=torch.uint8, device=dev)
    s4 = torch.ones(4, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        fp8.fp8_linear_rowwise(q, q, s4, s4, out_kind=fp8.OUT_FP8)
    with pytest.raises(ValueError):
        fp8.fp8_linear_rowwise(q, q, s4[:3], s4)
    with pytest.raises(fp8.Fp8motError):
        fp8.fp8_quant_per_row(torch.zeros((4, 24), dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("engine", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_linear_rowwise_special_scales(engine):
    # per-row scales NaN (a NaN row), 0 (a zero row) and +Inf (an Inf row),
    # per-channel scales 0 and NaN: alpha[m, n] = fp32(s_x[m] * s_w[n]) and
    # y = fp32(acc * alpha) give NaN, signed infinities and zeros exactly
    # where the oracle's epilogue does (R-24); the rest meets the GEMM bar
    dev = device()
    M, N, K = 40, 48, 272
    rng = np.random.default_rng(60 + engine)
    qx = rng.integers(0, 256, (M, K), dtype=np.int64).astype(np.uint8)
    qw = rng.integers(0, 256, (N, K), dtype=np.int64).astype(np.uint8)
    qx[(qx & 0x7F) == 0x7F] = 0x7E
    qw[(qw & 0x7F) == 0x7F] = 0x7E
    sx = rng.uniform(0.01, 0.1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    sx[3], sx[5], sx[8] = np.nan, 0.0, np.inf
    sw[7], sw[11] = 0.0, np.nan
    d = lambda a: torch.from_numpy(a).to(dev)   # noqa: E731
    y32 = host_f32(fp8.fp8_linear_rowwise(d(qx), d(qw), d(sx), d(sw), out_kind=fp8.OUT_F32, accum=engine))
    yb = host_bits(fp8.fp8_linear_rowwise(d(qx), d(qw), d(sx), d(sw), accum=engine))
    S, A = gemm_exact(qx, qw)
    with np.errstate(invalid="ignore", over="ignore"):
        want = epilogue_rowwise_f32(S, sx, sw)
    assert np.array_equal(np.isnan(y32), np.isnan(want))
    inf = np.isinf(want)
    assert inf.any() and np.array_equal(y32[inf], want[inf])
    zero = want == 0
    assert zero.any() and np.all(y32[zero] == 0)
    fin = np.isfinite(want) & ~zero
    alpha = epilogue_rowwise_alpha(sx, sw).astype(np.float64)
    err = np.abs(y32[fin].astype(np.float64) - alpha[fin] * S[fin])
    bound = 1e-5 * A
    if engine != fp8.ACC_EXACT:
        bound = bound + fp8_mfma_group_bound(qx, qw)
    assert np.all(err <= alpha[fin] * bound[fin])
    bits_nan = (yb & 0x7FFF) > 0x7F80
    assert np.array_equal(bits_nan, np.isnan(want))
    assert np.array_equal(yb[~bits_nan], f32_to_bf16(y32)[~bits_nan])
