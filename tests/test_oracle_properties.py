"""Property-based pins of the oracle (hypothesis; CPU): each property follows
from the mathematics of the format or the operation, not from the oracle's
own code, so a mistake in the oracle (a wrong tie rule, a dropped term, a
transposed operand, a sign lost) fails one of them on some input.

* E4M3 encoding (model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN ...",
  "Scheme": FP8 E4M3; the rounding readings of the oracle's formats module):
  the code is the nearest of the finite values, found here by a plain search
  over the values rebuilt from the format's definition, ties to the even
  code, saturating at 448.
* Static quantization: odd symmetry (negating the input flips only the sign
  bit) and monotonicity in the value and in the scale.
* The exact GEMM: splitting K into two blocks adds exactly (the sums are
  exact), swapping the operands transposes, and a single nonzero term gives
  that product.
* The observers: the max observer is order-free; the moving average stays
  within the range of the per-call maxima it has seen.
"""

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.formats import e4m3_decode, e4m3_encode, f32_to_bf16
from oracle.linear import gemm_exact, quant_static
from oracle.observer import (OBS_MAX, OBS_MOVING_AVG, ObserverState, call_amax,
                             observe)


def _finite_magnitudes():
    # E4M3FN from its definition: bias 7, three mantissa bits, exponent
    # field 0 subnormal (m * 2^-9), S.1111.111 NaN, everything else normal
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)   # index = the code's low 7 bits


MAGS = _finite_magnitudes()


def _encode_by_search(v):
    """Nearest finite E4M3 code of a float by exhaustive search, ties to the
    even code, saturating at 448; NaN -> 0x7F; the sign bit kept."""
    if np.isnan(v):
        return 0x7F
    sign = 0x80 if np.signbit(v) else 0
    a = abs(v)
    if a >= 448.0:
        return sign | 0x7E
    d = np.abs(MAGS - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
    return sign | code


f32 = st.floats(width=32, allow_nan=True, allow_infinity=True)
in_range = st.floats(min_value=-480.0, max_value=480.0, width=32)
# values a few float32 ulps around the midpoint between two neighbouring codes
near_mid = st.tuples(st.integers(0, 125), st.integers(-3, 3), st.booleans()).map(
    lambda t: (-1 if t[2] else 1) * float(np.nextafter(
        np.float32((MAGS[t[0]] + MAGS[t[0] + 1]) / 2),
        np.float32(np.inf if t[1] > 0 else -np.inf)) if t[1] else np.float32((MAGS[t[0]] + MAGS[t[0] + 1]) / 2))
    if abs(t[1]) <= 1 else (-1 if t[2] else 1) * float(
        np.float32((MAGS[t[0]] + MAGS[t[0] + 1]) / 2) * np.float32(1 + t[1] * 2.0 ** -23)))


@settings(max_examples=3000, deadline=None, derandomize=True)
@given(st.one_of(f32, in_range, near_mid))
def test_encode_is_the_nearest_code_by_search(v):
    x = np.float32(v)
    assert int(e4m3_encode(np.array([x]))[0]) == _encode_by_search(float(x))


@settings(max_examples=500, deadline=None, derandomize=True)
@given(st.lists(st.floats(min_value=-600.0, max_value=600.0, width=32), min_size=2, max_size=64))
def test_encode_is_monotone_and_decodes_within_half_a_step(vals):
    x = np.sort(np.array(vals, np.float32))
    dec = e4m3_decode(e4m3_encode(x))
    assert np.all(np.diff(dec) >= 0)
    inside = np.abs(x) < 448
    # the nearest value is at most half the gap to its neighbour away; the
    # largest gap below 448 is 32 (between 416 and 448), the smallest 2^-9
    a = np.abs(x[inside]).astype(np.float64)
    lo = np.searchsorted(MAGS, a, side="right") - 1          # the codes around |x|
    gap = MAGS[np.minimum(lo + 1, len(MAGS) - 1)] - MAGS[lo]
    assert np.all(np.abs(dec[inside] - x[inside]) <= gap / 2)


bf16_bits = st.integers(0, 0xFFFF)
scales = st.floats(min_value=2.0 ** -20, max_value=1024.0, width=32)


@settings(max_examples=400, deadline=None, derandomize=True)
@given(st.lists(bf16_bits, min_size=1, max_size=64), scales)
def test_quantize_is_odd_and_monotone(bits, s):
    x = np.array(bits, np.uint16)
    s = np.float32(s)
    q = quant_static(x, s)
    qn = quant_static(x ^ np.uint16(0x8000), s)
    vals = (x.astype(np.uint32) << 16).view(np.float32)
    ok = ~np.isnan(vals)
    assert np.array_equal(qn[ok], q[ok] ^ 0x80)          # negation flips the sign bit only
    assert np.all(q[~ok] == 0x7F) and np.all(qn[~ok] == 0x7F)
    order = np.argsort(vals[ok], kind="stable")
    dq = e4m3_decode(q[ok][order])
    assert np.all(np.diff(dq) >= 0)                      # monotone in the value


@settings(max_examples=300, deadline=None, derandomize=True)
@given(st.lists(bf16_bits, min_size=1, max_size=64), scales, scales)
def test_quantize_magnitude_does_not_grow_with_the_scale(bits, s1, s2):
    x = np.array(bits, np.uint16)
    x = x[~np.isnan((x.astype(np.uint32) << 16).view(np.float32))]
    lo, hi = sorted((np.float32(s1), np.float32(s2)))
    a_lo = np.abs(e4m3_decode(quant_static(x, lo)))
    a_hi = np.abs(e4m3_decode(quant_static(x, hi)))
    assert np.all(a_hi <= a_lo)


finite_codes = st.integers(0, 255).filter(lambda c: (c & 0x7F) != 0x7F)


FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(st.integers(1, 5), st.integers(1, 5), st.integers(1, 6), st.integers(1, 5),
       st.integers(0, 2 ** 32 - 1), st.sampled_from(["all", "extremes"]))
def test_gemm_blocks_of_k_add_exactly_and_transpose(M, N, k1, k2, seed, mix):
    K1, K2 = 16 * k1, 16 * k2
    rng = np.random.default_rng(seed)
    # every finite code, or only the largest and smallest magnitudes (the
    # sums then span the widest range of binades)
    pool = FINITE if mix == "all" else np.array([0x01, 0x81, 0x02, 0x7E, 0xFE, 0x7D, 0x00, 0x80], np.uint8)
    qa = rng.choice(pool, (M, K1 + K2))
    qb = rng.choice(pool, (N, K1 + K2))
    S, A = gemm_exact(qa, qb)
    S1, A1 = gemm_exact(qa[:, :K1], qb[:, :K1])
    S2, A2 = gemm_exact(qa[:, K1:], qb[:, K1:])
    assert np.array_equal(S, S1 + S2) and np.array_equal(A, A1 + A2)
    St, At = gemm_exact(qb, qa)
    assert np.array_equal(St, S.T) and np.array_equal(At, A.T)
    assert np.all(A >= np.abs(S))


@settings(max_examples=300, deadline=None, derandomize=True)
@given(finite_codes, finite_codes, st.integers(0, 31), st.integers(1, 3))
def test_gemm_single_term_is_the_product(ca, cb, k, blocks):
    K = 32 * blocks
    qa = np.zeros((1, K), np.uint8)
    qb = np.zeros((1, K), np.uint8)
    qa[0, k], qb[0, k] = ca, cb
    S, A = gemm_exact(qa, qb)
    p = float(e4m3_decode(ca)) * float(e4m3_decode(cb))
    assert S[0, 0] == p and A[0, 0] == abs(p)


amaxes = st.lists(st.floats(min_value=0.0, max_value=1e4, width=32), min_size=1, max_size=40)


@settings(max_examples=300, deadline=None, derandomize=True)
@given(amaxes, st.randoms())
def test_max_observer_is_order_free_and_moving_average_stays_in_range(a, rnd):
    def run(seq, mode):
        s = ObserverState()
        for v in seq:
            observe(s, v, mode, 0.01)
        return np.float32(s.m)
    shuffled = list(a)
    rnd.shuffle(shuffled)
    assert run(a, OBS_MAX) == run(shuffled, OBS_MAX) == np.float32(max(a))
    m = run(a, OBS_MOVING_AVG)
    assert np.float32(min(a)) <= m <= np.float32(max(a))


@settings(max_examples=200, deadline=None, derandomize=True)
@given(st.lists(st.floats(min_value=-1e4, max_value=1e4, width=32), min_size=1, max_size=64))
def test_call_amax_is_the_largest_magnitude(vals):
    x = f32_to_bf16(np.array(vals, np.float32))
    dec = (x.astype(np.uint32) << 16).view(np.float32)
    assert call_amax(x) == np.max(np.abs(dec))
