"""Pins for oracle.linear: quantize, RTN weights, exact GEMM, epilogues,
re-quantization failure mode and the shared-scale check."""

import fractions
import json
import os

import numpy as np
import torch

from oracle.formats import (E4M3_TABLE, bf16_to_f32, e4m3_decode, e4m3_encode,
                            f32_to_bf16)
from oracle.linear import (check_shared_scale, epilogue_bf16, epilogue_f32,
                           epilogue_fp8, gemm_exact, gemm_f32acc, quant_static,
                           requantize_onto_max, rtn_weight, scale_from_amax)

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")


def torch_e4m3(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_quant_static_all_bf16_against_torch():
    x = bf16_to_f32(ALL_BF16)
    for s in (np.float32(1.0), np.float32(0.0123), np.float32(20.0 / 448),
              np.float32(3.7e-3), np.float32(1.337)):
        ours = quant_static(ALL_BF16, s)
        with np.errstate(all="ignore"):
            q = (torch.from_numpy(x) / torch.tensor(s)).numpy()
        inrange = np.abs(q) <= 464
        assert np.array_equal(ours[inrange], torch_e4m3(q[inrange]))
        fin = np.isfinite(q) & ~inrange
        assert np.all((ours[fin] & 0x7F) == 0x7E)
        assert np.all(ours[np.isnan(q)] == 0x7F)


def test_quant_static_power_of_two_scale_is_pure_encode():
    x = bf16_to_f32(ALL_BF16)
    for k in (-12, -3, 0, 5):
        s = np.float32(2.0 ** k)
        with np.errstate(invalid="ignore"):
            ref = e4m3_encode(np.ldexp(x.astype(np.float64), -k))
        assert np.array_equal(quant_static(ALL_BF16, s), ref)


def test_quant_static_idempotent_on_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    rng = np.random.default_rng(3)
    for s in rng.uniform(1e-4, 10, 20).astype(np.float32):
        # enc(fp32(fp32(dec(q) * s) / s)) == q: two float32 roundings move a
        # code's value by ~2^-23 relative, far from any E4M3 midpoint
        v = (e4m3_decode(codes).astype(np.float32) * s).astype(np.float32)
        q = e4m3_encode((v / s).astype(np.float32))
        assert np.array_equal(q, codes)


def test_rtn_weight_roundtrip_bound_and_no_saturation():
    rng = np.random.default_rng(4)
    w = torch.from_numpy(rng.standard_normal((256, 512)).astype(np.float32) * 0.02)
    wb = w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = rtn_weight(wb)
    wf = bf16_to_f32(wb).astype(np.float64)
    amax = np.max(np.abs(wf))
    assert s == np.float32(np.float32(amax) / np.float32(448))
    r = e4m3_decode(q) * np.float64(s)
    err = np.abs(wf - r)
    a = np.abs(wf / np.float64(s))
    normal = a >= 2.0 ** -6
    bound = np.where(normal,
                     np.float64(s) * 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 4),
                     np.float64(s) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    # the amax element lands on +-448 and nothing saturates beyond it
    i = np.argmax(np.abs(wf))
    assert (q.ravel()[i] & 0x7F) == 0x7E
    assert np.count_nonzero((q & 0x7F) == 0x7F) == 0


def _int_gemm(qa, qb):
    """Exact integer reference: products scaled by 2^18 are integers."""
    ia = np.round(e4m3_decode(qa) * 2 ** 9).astype(np.int64)
    ib = np.round(e4m3_decode(qb) * 2 ** 9).astype(np.int64)
    assert np.array_equal(ia / 2 ** 9, e4m3_decode(qa))
    return ia @ ib.T


def _random_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E      # no NaN codes in GEMM operands
    return c


def test_gemm_exact_against_integer_arithmetic():
    rng = np.random.default_rng(5)
    for (M, N, K) in [(7, 5, 16), (33, 17, 512), (64, 48, 4096)]:
        qa = _random_codes(rng, (M, K))
        qb = _random_codes(rng, (N, K))
        S, A = gemm_exact(qa, qb)
        I = _int_gemm(qa, qb)
        assert np.array_equal(S * 2 ** 18, I.astype(np.float64))
        assert np.array_equal((S * 2 ** 18).astype(np.int64), I)
        IA = np.abs(np.round(e4m3_decode(qa) * 2 ** 9)).astype(np.int64) @ \
            np.abs(np.round(e4m3_decode(qb) * 2 ** 9)).astype(np.int64).T
        assert np.array_equal((A * 2 ** 18).astype(np.int64), IA)


def test_gemm_exact_adversarial_magnitudes():
    # 448^2 terms and 2^-18 terms in one sum: exact only with enough bits
    K = 8192
    qa = np.zeros((2, K), np.uint8)
    qb = np.zeros((2, K), np.uint8)
    qa[:, ::2] = 0x7E
    qb[:, ::2] = 0x7E
    qa[:, 1::2] = 0x01
    qb[:, 1::2] = 0x01
    qb[1, ::4] = 0xFE
    S, _ = gemm_exact(qa, qb)
    ref = fractions.Fraction(0)
    for k in range(K):
        ref += fractions.Fraction(float(E4M3_TABLE[qa[0, k]])) * \
            fractions.Fraction(float(E4M3_TABLE[qb[1, k]]))
    assert fractions.Fraction(float(S[0, 1])) == ref
    assert S[0, 0] == (K // 2) * 448.0 ** 2 + (K // 2) * 2.0 ** -18


def test_gemm_exact_tiny_bruteforce_fractions():
    rng = np.random.default_rng(6)
    qa = _random_codes(rng, (3, 16))
    qb = _random_codes(rng, (4, 16))
    S, A = gemm_exact(qa, qb)
    for m in range(3):
        for n in range(4):
            s = sum(fractions.Fraction(float(E4M3_TABLE[qa[m, k]])) *
                    fractions.Fraction(float(E4M3_TABLE[qb[n, k]]))
                    for k in range(16))
            assert fractions.Fraction(float(S[m, n])) == s


def test_gemm_all_code_pairs_single_term():
    # every non-NaN code pair as a one-term dot product (K = 16, k = 0 only)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    qa = np.zeros((254, 16), np.uint8)
    qb = np.zeros((254, 16), np.uint8)
    qa[:, 0] = codes
    qb[:, 0] = codes
    S, A = gemm_exact(qa, qb)
    v = E4M3_TABLE[codes]
    assert np.array_equal(S, np.outer(v, v))
    assert np.array_equal(A, np.abs(np.outer(v, v)))
    # every product has a 4-bit x 4-bit significand: exact in BF16
    y = epilogue_bf16(S, 1.0, 1.0)
    assert np.array_equal(bf16_to_f32(y).astype(np.float64), np.outer(v, v))


def test_gemm_identity_weight_gives_decoded_input():
    rng = np.random.default_rng(7)
    qx = _random_codes(rng, (37, 64))
    eye = np.zeros((64, 64), np.uint8)
    eye[np.arange(64), np.arange(64)] = 0x38
    S, _ = gemm_exact(qx, eye)
    assert np.array_equal(S, e4m3_decode(qx))


def test_f32_accumulation_within_tolerance_of_exact():
    rng = np.random.default_rng(8)
    qa = _random_codes(rng, (64, 2048))
    qb = _random_codes(rng, (64, 2048))
    S, A = gemm_exact(qa, qb)
    F = gemm_f32acc(qa, qb).astype(np.float64)
    assert np.all(np.abs(F - S) <= 1e-5 * A)


def test_epilogues_against_torch_casts():
    rng = np.random.default_rng(9)
    S = rng.standard_normal((50, 60)) * 1e4
    sx, sw, sy = np.float32(0.0213), np.float32(1.7e-4), np.float32(0.011)
    alpha = np.float32(sx * sw)
    y32 = epilogue_f32(S, sx, sw)
    ref32 = (torch.from_numpy(S.astype(np.float32)) * torch.tensor(alpha)).numpy()
    assert np.array_equal(y32, ref32)
    yb = epilogue_bf16(S, sx, sw)
    refb = torch.from_numpy(ref32).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(yb, refb.view(np.uint16))
    y8 = epilogue_fp8(S, sx, sw, sy)
    q = (torch.from_numpy(ref32) / torch.tensor(sy)).numpy()
    inr = np.abs(q) <= 464
    assert np.array_equal(y8[inr], torch_e4m3(q[inr]))
    assert np.all((y8[~inr] & 0x7F) == 0x7E)


def test_requantization_failure_mode():
    rng = np.random.default_rng(10)
    ws = [torch.from_numpy(rng.standard_normal((64, 256)).astype(np.float32) * sd)
          .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
          for sd in (0.02, 0.013, 0.031)]
    qs, ss = zip(*[rtn_weight(w) for w in ws])
    # the test can only discriminate if the group's scales really differ
    assert len(set(float(s) for s in ss)) == 3
    rq, smax = requantize_onto_max(qs, ss)
    for q, s, r in zip(qs, ss, rq):
        changed = np.count_nonzero(q != r)
        if s == smax:
            assert changed == 0
        else:
            assert changed > 0
    # power-of-two ratio: a member's values are divided exactly by 4, so only
    # codes whose quarter falls below the smallest normal (2^-6) can lose value
    s0 = np.float32(0.01)
    q0 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    (r0, r1), _ = requantize_onto_max([q0, q0], [s0, np.float32(4 * s0)])
    exact = e4m3_decode(q0) / 4
    assert np.array_equal(r1, q0)
    lost = e4m3_decode(r0) != exact
    assert lost.any()
    assert np.all(np.abs(exact[lost]) < 2.0 ** -6)


def test_check_shared_scale():
    a = np.float32(0.0123)
    assert check_shared_scale([a, a, a])
    assert not check_shared_scale([a, np.nextafter(a, np.float32(1))])
    assert not check_shared_scale([a, np.float32(np.nan)])
    assert not check_shared_scale([np.float32(0), np.float32(0)])
    assert not check_shared_scale([np.float32(-1)])
    assert not check_shared_scale([np.float32(np.inf)])
    assert not check_shared_scale([])


def test_scale_from_amax_is_single_division():
    for a in (1.0, 20.5, 3.1e-5, 448.0):
        assert scale_from_amax(a) == np.float32(np.float32(a) / np.float32(448))
    assert scale_from_amax(448.0) == 1.0


def test_group_counts_reading():
    # Pull request "Description" and "What changed": Nano's formerly fused
    # groups per layer are gen QKV (3 shards), und gate/up (2) and gen gate/up
    # (2): 7 shards and 3 groups per layer, at most 4 of them not holding the
    # group's max scale.  The printed counts (tests/golden) must fit that
    # structure: 36 layers -> 252 shards, 108 groups, <= 144 changed; 64
    # layers -> 448 shards, 192 groups, <= 256 changed; ~56% in both.
    g = json.load(open(GOLDEN))["requantization_failure"]
    for name, layers in (("nano", 36), ("super", 64)):
        c = g[name]
        assert 7 * layers == c["fused_shards"] and 3 * layers == c["groups"]
        assert c["affected_shards"] <= 4 * layers
        assert round(100 * c["affected_shards"] / c["fused_shards"]) == g["affected_percent_printed"]
