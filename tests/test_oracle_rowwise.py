"""Pins for oracle.rowwise (per-channel weight / per-token activation FP8;
model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN + moving-average activation
observer", section 3.2)."""

import numpy as np
import torch

from oracle.formats import bf16_to_f32, e4m3_decode
from oracle.linear import amax_f32, gemm_exact, quant_static, scale_from_amax
from oracle.rowwise import (epilogue_rowwise_bf16, epilogue_rowwise_f32,
                            quant_per_row, row_scales, rtn_weight_per_channel)
from mlp_fp8_quant_amd import workloads


def _bf16(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


def test_single_row_is_the_per_tensor_quantization():
    rng = np.random.default_rng(41)
    x = _bf16(rng.standard_normal((1, 777)) * 5)
    codes, s = quant_per_row(x)
    s_t = scale_from_amax(amax_f32(x))
    assert s[0] == s_t
    assert np.array_equal(codes[0], quant_static(x[0], s_t))


def test_row_scale_against_torch_amax():
    rng = np.random.default_rng(42)
    x = _bf16(rng.standard_normal((37, 300)) * rng.uniform(0.01, 50, (37, 1)))
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    want = (t.abs().amax(dim=1) / 448.0).numpy().astype(np.float32)
    assert np.array_equal(row_scales(x), want)


def test_power_of_two_row_rescaling_keeps_codes():
    # scaling one row by 2^k scales its scale by 2^k and keeps its codes; a
    # single per-tensor scale would change the codes of the smaller rows
    rng = np.random.default_rng(43)
    base = rng.standard_normal(512).astype(np.float32)
    rows = np.stack([base * np.float32(2.0 ** k) for k in (-6, 0, 3, 9)])
    x = _bf16(rows)
    codes, s = quant_per_row(x)
    for r in range(1, 4):
        assert np.array_equal(codes[r], codes[0])
    assert np.array_equal(s / s[0], np.float32([1, 2 ** 6, 2 ** 9, 2 ** 15]))
    per_tensor = quant_static(x, scale_from_amax(amax_f32(x)))
    assert not np.array_equal(per_tensor[0], codes[0])


def test_every_nonzero_row_reaches_448():
    rng = np.random.default_rng(44)
    x = _bf16(rng.standard_normal((64, 129)) * rng.uniform(1e-3, 1e3, (64, 1)))
    codes, _ = quant_per_row(x)
    assert np.all(np.max(codes & 0x7F, axis=1) == 0x7E)


def test_zero_nan_and_inf_rows():
    x = _bf16([[0.0, -0.0, 0.0, -0.0],
               [1.0, np.nan, -2.0, 0.5],
               [1.0, np.inf, -2.0, 0.0],
               [3.0, -1.5, 0.75, 448.0]])
    codes, s = quant_per_row(x)
    assert s[0] == 0 and list(codes[0]) == [0x00, 0x80, 0x00, 0x80]
    assert np.isnan(s[1]) and np.all(codes[1] == 0x7F)
    assert np.isinf(s[2]) and list(codes[2]) == [0x00, 0x7F, 0x80, 0x00]
    assert s[3] == np.float32(448.0 / 448.0)
    assert list(e4m3_decode(codes[3])) == [3.0, -1.5, 0.75, 448.0]


def test_rowwise_epilogue_is_the_scaled_dequantized_product():
    # y[m, n] ~= sum_k (s_x[m] dec(qx)) (s_w[n] dec(qw)) in float64: a scale
    # applied to the wrong axis (M != N, distinct scales) fails
    rng = np.random.default_rng(45)
    x = _bf16(rng.standard_normal((24, 96)) * rng.uniform(0.1, 10, (24, 1)))
    w = _bf16(rng.standard_normal((40, 96)) * rng.uniform(0.005, 0.05, (40, 1)))
    qx, sx = quant_per_row(x)
    qw, sw = rtn_weight_per_channel(w)
    S, A = gemm_exact(qx, qw)
    y32 = epilogue_rowwise_f32(S, sx, sw)
    ref = (e4m3_decode(qx) * sx[:, None].astype(np.float64)) @ \
          (e4m3_decode(qw) * sw[:, None].astype(np.float64)).T
    bound = 4 * 2.0 ** -24 * (A * sx[:, None].astype(np.float64) * sw[None, :]) + 1e-300
    assert np.all(np.abs(y32 - ref) <= bound + 2.0 ** -23 * np.abs(ref))
    # against the BF16 model it approximates: within FP8 quantization error
    yb = bf16_to_f32(epilogue_rowwise_bf16(S, sx, sw)).astype(np.float64)
    full = bf16_to_f32(x).astype(np.float64) @ bf16_to_f32(w).astype(np.float64).T
    assert np.max(np.abs(yb - full)) < 0.08 * np.max(np.abs(full))


def test_empty_rows_scale_as_zero_rows():
    # appending zeros to a row never changes its amax, so an empty row (K = 0)
    # takes the scale of a zero row of any length: 0
    _, s_empty = quant_per_row(np.zeros((3, 0), np.uint16))
    for K in (16, 48):
        q, s = quant_per_row(np.zeros((3, K), np.uint16))
        assert np.array_equal(s.view(np.uint32), s_empty.view(np.uint32))
        assert np.all(q == 0)
    x = _bf16(np.random.default_rng(4).standard_normal((3, 32)))
    _, s_x = quant_per_row(x)
    _, s_pad = quant_per_row(np.concatenate([x, np.zeros((3, 16), np.uint16)], axis=1))
    assert np.array_equal(s_x.view(np.uint32), s_pad.view(np.uint32))
