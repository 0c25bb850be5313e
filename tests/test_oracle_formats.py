"""Pins for oracle.formats against the E4M3/BF16 definitions and torch casts.

torch's CPU casts to float8_e4m3fn and bfloat16 are independent library
routines: round to nearest even, with float8 overflow going to NaN instead of
saturating, so they pin the oracle wherever |x| <= 464 (the tie point between
448 and the next, non-existent, step 480).
"""

import numpy as np
import pytest
import torch

from oracle.formats import (E4M3_TABLE, bf16_to_f32, bf16_ulps, e4m3_decode,
                            e4m3_encode, e4m3_steps, f32_to_bf16)


def torch_e4m3(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_table_closed_form():
    t = E4M3_TABLE
    nan = np.isnan(t)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.count_nonzero(~nan) == 254
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)      # code order == magnitude order
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = e4m3_decode(np.arange(256, dtype=np.uint8))
    same = (ref.astype(np.float64) == ours) | (np.isnan(ref) & np.isnan(ours))
    assert same.all()


def test_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    v = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(v), codes)


def test_encode_midpoints_ties_to_even_and_neighbours():
    pos = E4M3_TABLE[:127]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    lo = np.arange(126)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(e4m3_encode(mid), even.astype(np.uint8))
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(e4m3_encode(below), lo.astype(np.uint8))
    assert np.array_equal(e4m3_encode(above), (lo + 1).astype(np.uint8))
    # and the same with the sign bit
    assert np.array_equal(e4m3_encode(-mid), (even | 0x80).astype(np.uint8))


def test_encode_saturation_nan_and_signed_zero():
    big = np.array([448, 448.5, 463.9, 464, 464.1, 480, 1e4, 3e38, np.inf],
                   np.float32)
    assert np.all(e4m3_encode(big) == 0x7E)
    assert np.all(e4m3_encode(-big) == 0xFE)
    assert e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F
    assert e4m3_encode(np.array([-np.nan], np.float32))[0] == 0x7F
    assert e4m3_encode(np.array([0.0], np.float32))[0] == 0x00
    assert e4m3_encode(np.array([-0.0], np.float32))[0] == 0x80
    tiny = np.array([2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45], np.float32)
    assert np.all(e4m3_encode(tiny) == 0x00)       # 2^-10 is a tie -> even 0
    assert np.all(e4m3_encode(-tiny) == 0x80)
    just = np.nextafter(np.float32(2.0 ** -10), np.float32(1))
    assert e4m3_encode(np.array([just]))[0] == 0x01


def _sweep_patterns(step, lo_bits, hi_bits):
    return np.arange(lo_bits, hi_bits, step, dtype=np.uint64).astype(np.uint32)


def test_encode_matches_torch_sweep():
    # every 61st FP32 pattern from +0 up to 464, plus every pattern in the
    # binade [2^-7, 2^-6) (subnormal/normal boundary) and [256, 464]
    hi = int(np.float32(464).view(np.uint32)) + 1
    parts = [
        _sweep_patterns(61, 0, hi),
        _sweep_patterns(1, int(np.float32(2.0 ** -7).view(np.uint32)),
                        int(np.float32(2.0 ** -6).view(np.uint32)) + 1),
        _sweep_patterns(1, int(np.float32(256.0).view(np.uint32)), hi),
    ]
    bits = np.concatenate(parts)
    x = bits.view(np.float32)
    for sgn in (1.0, -1.0):
        v = (x * np.float32(sgn)).astype(np.float32)
        ours = e4m3_encode(v)
        ref = torch_e4m3(v)
        assert np.array_equal(ours, ref), np.nonzero(ours != ref)[0][:5]


def test_encode_monotone():
    x = np.sort(np.random.default_rng(1).uniform(-500, 500, 200_000)
                .astype(np.float32))
    vals = e4m3_decode(e4m3_encode(x))
    assert np.all(np.diff(vals) >= 0)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    # force ties and near-ties in the low half
    bits[::4] = (bits[::4] & 0xFFFF0000) | 0x8000
    bits[1::4] = (bits[1::4] & 0xFFFF0000) | 0x7FFF
    bits[2::4] = (bits[2::4] & 0xFFFF0000) | 0x8001
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    ours = f32_to_bf16(x)
    ref = torch_bf16(x)
    assert np.array_equal(ours[finite], ref[finite])
    nan = np.isnan(x)
    assert np.all((ours[nan] & 0x7FFF) == 0x7FC0)
    inf = np.array([np.inf, -np.inf], np.float32)
    assert np.array_equal(f32_to_bf16(inf), torch_bf16(inf))


def test_bf16_to_f32_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_step_and_ulp_distances():
    assert e4m3_steps(np.uint8(0x01), np.uint8(0x80)) == 1
    assert e4m3_steps(np.uint8(0x00), np.uint8(0x80)) == 0
    assert e4m3_steps(np.uint8(0x7E), np.uint8(0x7D)) == 1
    assert e4m3_steps(np.uint8(0x81), np.uint8(0x01)) == 2
    assert bf16_ulps(np.uint16(0x8000), np.uint16(0x0000)) == 0
    assert bf16_ulps(np.uint16(0x3F80), np.uint16(0x3F81)) == 1
