"""Number formats: OCP E4M3FN (the FP8 of the FP8 checkpoints) and BF16.

Model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN ...", section "Scheme": both
weights and activations are FP8 E4M3 with one scale per tensor.  The pages do
not spell out the bit format; this oracle takes the OCP E4M3FN definition
(bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite
magnitude 448), which is the format whose maximum the workload descriptions
state (448).

Readings where the pages are silent:

* rounding is to nearest, ties to the even code (the card says "RTN" and
  "compress rounding" without a tie rule);
* overflow saturates to +-448 (the moving-average scale is said to *clip* the
  rarest activations, so an overflowing activation must clip, not become NaN);
  +-Inf saturates as well;
* NaN encodes to the canonical 0x7F;
* the sign of zero is kept: -0 and negative values that round to zero give
  0x80.
"""

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def _decode_one(code: int) -> float:
    """Value of one E4M3FN code, straight from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        # subnormal: m * 2^(1 - bias - 3) = m * 2^-9
        return sign * m * 2.0 ** -9
    # normal: (1 + m/8) * 2^(e - 7) = (8 + m) * 2^(e - 10)
    return sign * (8 + m) * 2.0 ** (e - 10)


#: float64 value of each of the 256 codes (NaN for 0x7F and 0xFF).
E4M3_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes in code order: code c (0..126) has value
# _POS[c].  They are strictly increasing, which the encoder relies on.
_POS = E4M3_TABLE[:127].copy()
# Midpoint between consecutive magnitudes (exact: dyadic numbers with a few
# significant bits).
_MID = (_POS[:-1] + _POS[1:]) / 2.0


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 E4M3 codes to float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3_TABLE[codes]


def e4m3_encode(v) -> np.ndarray:
    """Encode real values to E4M3 codes: nearest finite value, ties to even.

    ``v`` may be float32 or float64; each element's exact value is encoded
    (callers that specify a float32 intermediate round to float32 first).
    Magnitudes at or above 448, and infinities, saturate to 0x7E with the
    input's sign; NaN gives 0x7F; zero and underflow keep the sign bit.
    """
    v = np.asarray(v)
    if v.dtype not in (np.float32, np.float64):
        raise TypeError("e4m3_encode takes float32 or float64 input")
    x = v.astype(np.float64)  # exact widening
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    # lo: largest code whose magnitude is <= a (codes 0..126)
    lo = np.searchsorted(_POS, a, side="right") - 1
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    mid = _MID[np.minimum(lo, 125)]
    pick_hi = a > mid
    tie = a == mid
    # a tie goes to the even code; codes lo and lo+1 differ in their last bit
    pick_hi = pick_hi | (tie & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)  # saturate (also +-Inf)
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    code = np.where(nan, NAN_CODE, code).astype(np.uint8)
    return code


# ---------------------------------------------------------------------------
# BF16
# ---------------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) to float32: the upper half of an FP32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """Round float32 to BF16 bit patterns, to nearest with ties to even.

    The low 16 bits of the FP32 pattern are the part dropped; adding
    0x7FFF plus the kept LSB and truncating is round-half-to-even on the
    magnitude.  NaN becomes the canonical quiet NaN 0x7FC0 (sign kept).
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
    r = np.where(nan, sign | np.uint16(0x7FC0), r)
    return r.astype(np.uint16)


def e4m3_steps(a, b) -> np.ndarray:
    """Ordinal distance between E4M3 codes on the sign-magnitude line.

    Codes are mapped to integers with +0 and -0 both at 0, positive codes at
    their magnitude index and negative codes at minus it; e.g. 2^-9 (0x01)
    and -0 (0x80) are one step apart.  NaN codes map to a far sentinel.
    """
    def ordv(c):
        c = np.asarray(c, dtype=np.int64)
        mag = c & 0x7F
        o = np.where(c & 0x80, -mag, mag)
        return np.where(mag == 0x7F, 1 << 20, o)
    return np.abs(ordv(a) - ordv(b))


def bf16_ulps(a, b) -> np.ndarray:
    """Ordinal distance between BF16 patterns (same mapping as e4m3_steps)."""
    def ordv(c):
        c = np.asarray(c, dtype=np.int64)
        mag = c & 0x7FFF
        return np.where(c & 0x8000, -mag, mag)
    return np.abs(ordv(a) - ordv(b))
