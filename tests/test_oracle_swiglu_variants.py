"""Pins for the SwiGLU variants of oracle.swiglu: alpha (a gain inside the
sigmoid), beta (an offset on up) and the one-input form with gate and up
adjacent in one tensor (pull request "Load static FP8 Cosmos3 Nano/Super
checkpoints without re-quantizing them", the commit messages on
swiglu_alpha / swiglu_beta and on silu_and_mul_2in)."""

import numpy as np
import pytest
import torch

from oracle.formats import bf16_to_f32, e4m3_encode
from oracle.swiglu import (silu_mul_ab_f64, silu_mul_ab_fp8,
                           silu_mul_adjacent_fp8, silu_mul_f64,
                           silu_mul_fp8, split_adjacent)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_alpha_zero_is_half_gate_closed_form():
    # sigmoid(0) = 1/2 exactly: h = g * (u + beta) / 2 for every g
    g = _bf16([3.0, -5.0, 0.5, 96.0])
    u = _bf16([2.0, 7.0, -4.0, 0.25])
    h = silu_mul_ab_f64(g, u, alpha=0.0, beta=1.5)
    expect = np.array([3.0 * 3.5 / 2, -5.0 * 8.5 / 2, 0.5 * -2.5 / 2, 96.0 * 1.75 / 2])
    assert np.array_equal(h, expect)


def test_gain_inside_sigmoid_odd_identity():
    # f(g) = g sigmoid(a g) satisfies f(g) - f(-g) = g (sigmoid(x) + sigmoid(-x)
    # = 1); a gain applied outside the sigmoid, or to u, breaks it
    rng = np.random.default_rng(21)
    g = _bf16(rng.standard_normal(4096) * 3)
    ones = _bf16(np.ones(4096))
    for a in (1.702, 0.37, 4.0):
        f_pos = silu_mul_ab_f64(g, ones, alpha=a)
        f_neg = silu_mul_ab_f64(_bf16(-bf16_to_f32(g)), ones, alpha=a)
        assert np.allclose(f_pos - f_neg, bf16_to_f32(g).astype(np.float64), rtol=0, atol=1e-12)


def test_large_gain_tends_to_relu():
    # a -> inf: g sigmoid(a g) -> max(g, 0)
    g = _bf16([2.0, -2.0, 0.75, -0.75])
    u = _bf16([1.0, 1.0, 1.0, 1.0])
    h = silu_mul_ab_f64(g, u, alpha=1e4)
    assert np.array_equal(h, [2.0, 0.0, 0.75, 0.0])


def test_beta_is_an_offset_on_up_only():
    rng = np.random.default_rng(22)
    g = _bf16(rng.standard_normal(1000) * 2)
    u = _bf16(rng.standard_normal(1000) * 2)
    gf = bf16_to_f32(g).astype(np.float64)
    uf = bf16_to_f32(u).astype(np.float64)
    h = silu_mul_ab_f64(g, u, alpha=1.0, beta=1.0)
    # against torch's SiLU on the gate and a plain offset on up
    ref = torch.nn.functional.silu(torch.from_numpy(gf)).numpy() * (uf + 1.0)
    assert np.allclose(h, ref, rtol=1e-14, atol=0)


def test_defaults_are_plain_swiglu_bitwise():
    rng = np.random.default_rng(23)
    g = _bf16(np.concatenate([rng.standard_normal(5000) * 4, [0.0, -0.0, 1.0, -1.0]]))
    u = _bf16(np.concatenate([rng.standard_normal(5000) * 4, [-0.0, -0.0, -0.0, 0.0]]))
    s = np.float32(0.0421)
    assert np.array_equal(silu_mul_ab_fp8(g, u, s), silu_mul_fp8(g, u, s))
    h = silu_mul_ab_f64(g, u)
    assert np.array_equal(np.signbit(h), np.signbit(silu_mul_f64(g, u)))


def test_swigluoai_shape_against_torch():
    # alpha = 1.702, beta = 1: x_glu * sigmoid(1.702 x_glu) * (x_lin + 1)
    rng = np.random.default_rng(24)
    g = _bf16(rng.standard_normal(20000) * 3)
    u = _bf16(rng.standard_normal(20000) * 3)
    s = np.float32(0.125)
    gf = torch.from_numpy(bf16_to_f32(g).astype(np.float64))
    uf = torch.from_numpy(bf16_to_f32(u).astype(np.float64))
    a = float(np.float32(1.702))
    h = gf * torch.sigmoid(a * gf) * (uf + 1.0)
    q = (h / float(s)).to(torch.float32)
    inr = q.abs() <= 448
    ref = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = silu_mul_ab_fp8(g, u, s, alpha=1.702, beta=1.0)
    assert inr.float().mean() > 0.99
    assert np.array_equal(ours[inr.numpy()], ref[inr.numpy()])
    assert np.all((ours[~inr.numpy()] & 0x7F) == 0x7E)   # beyond 448: saturated


def test_adjacent_layout_hand_example():
    # one row, I = 2: x = [g0, g1, u0, u1]; alpha = 0 makes sigmoid = 1/2, so
    # h = g (u + beta) / 2 = [2*4/2, 4*6/2] = [4, 12] -> codes at scale 1
    x = _bf16([[2.0, 4.0, 3.0, 5.0]])
    codes = silu_mul_adjacent_fp8(x, np.float32(1.0), alpha=0.0, beta=1.0)
    assert codes.shape == (1, 2)
    assert list(codes[0]) == list(e4m3_encode(np.array([4.0, 12.0], np.float32)))
    # gate taken from the second half would give [4.5, 12.5] -> different codes
    assert list(codes[0]) != list(e4m3_encode(np.array([4.5, 12.5], np.float32)))


def test_adjacent_equals_two_input_on_halves_and_rejects_odd():
    rng = np.random.default_rng(25)
    x = _bf16(rng.standard_normal((3, 5, 2 * 48)) * 3)
    g, u = split_adjacent(x)
    assert g.shape == (3, 5, 48) and u.shape == (3, 5, 48)
    assert np.array_equal(g, x[..., :48]) and np.array_equal(u, x[..., 48:])
    s = np.float32(0.02)
    assert np.array_equal(silu_mul_adjacent_fp8(x, s, 1.702, 1.0).ravel(),
                          silu_mul_ab_fp8(g, u, s, 1.702, 1.0))
    with pytest.raises(ValueError):
        split_adjacent(np.zeros((2, 7), np.uint16))
