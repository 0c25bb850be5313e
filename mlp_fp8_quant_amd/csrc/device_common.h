// Device helpers shared by the libfp8mot kernels (gfx950 only).
//
// Number formats follow the model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN
// + moving-average activation observer", section "Scheme": FP8 E4M3 weights
// and activations, one scale per tensor.  The E4M3 variant is OCP E4M3FN
// (bias 7, no infinities, S.1111.111 = NaN, largest finite 448).  Rounding is
// to nearest with ties to the even code; overflow saturates to +-448 so that
// an activation above the calibrated range is clipped; NaN becomes 0x7F and
// the sign of zero is kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mot {

// BF16 bit pattern -> FP32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two FP32 values -> two BF16 (round to nearest even) packed lo | hi << 16,
// with the gfx950 packed conversion.  For every non-NaN input it gives the
// integer rounding of the bit pattern, (u + 0x7FFF + bit 16 of u) >> 16,
// overflow to +-Inf included; a NaN stays a NaN.  fp8mot_convert_f32 runs it
// on any FP32 input so that a test can check it over all 2^32 patterns.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// FP32 -> E4M3FN code with integer round-to-nearest-even on the bit pattern.
//  |v| >= 448 (and Inf): saturate to 0x7E.
//  [2^-6, 448): keep exponent and 3 mantissa bits, RNE on the 20 dropped
//    bits; a carry moves into the exponent as it should; re-bias 127 -> 7.
//  below 2^-6: E4M3 subnormals are multiples of 2^-9; adding 2^14, whose
//    FP32 ulp is 2^-9, rounds |v| to that grid (RNE) in one addition, and
//    the integer difference of the bit patterns is the code (0..8, where 8
//    is the smallest normal, 0x08).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {
    code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - 0x3C0u;
  } else {
    const float f = __fadd_rn(__uint_as_float(a), 16384.0f);
    code = __float_as_uint(f) - 0x46800000u;
  }
  code |= (u >> 24) & 0x80u;
  return a > 0x7F800000u ? 0x7Fu : code;
}

// Four FP32 values -> four E4M3 codes packed little-endian in a dword, using
// the gfx950 conversion instruction.  A NaN-propagating clamp to [-448, 448]
// (IEEE-754 maximum / minimum) makes the conversion saturate and leaves NaN a
// NaN, which the conversion turns into 0xFF; no finite input gives 0xFF
// (-448 is 0xFE), so clearing the sign bit of every 0xFF byte yields 0x7F.
// A byte is 0xFF exactly when its low seven bits plus one carry into bit 7
// and its own bit 7 is set; the low-seven-bit sums cannot carry across
// bytes.  Over every FP32 bit pattern, NaN included, this gives the codes of
// e4m3_encode (fp8mot_convert_f32 runs both on any FP32 input; a test checks
// them over all 2^32 patterns).
__device__ __forceinline__ float clamp448(float v) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(v, -448.0f), 448.0f);
}
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), (int)w, true);
  const uint32_t nan_bytes = (((w & 0x7F7F7F7Fu) + 0x01010101u) & w) & 0x80808080u;
  return w ^ nan_bytes;
}

// x / s for the E4M3 encoder, bit for bit the IEEE quotient where it matters,
// in four operations instead of a full division (whose ~11 instructions per
// element made the quantize kernel partly VALU-bound).  Valid for a scale s
// in [2^-60, 2^60] with r = 1 / s (correctly rounded) and lim = 1024 * s:
//  * x is first clamped to +-lim (NaN-propagating): |x / s| > 1024 encodes
//    to +-448 either way, and the clamp keeps the steps below finite;
//  * q0 = x * r is within one ulp of x / s, the remainder e = x - q0 * s is
//    exact with an FMA, and q0 + e * r rounded once is the correctly rounded
//    quotient (Markstein's theorem: r correctly rounded, q0 within one ulp,
//    no step overflows or underflows -- which holds for |x / s| in
//    [2^-71, 1024] given the range of s);
//  * below that, the quotient underflows, the result stays far below the
//    smallest E4M3 subnormal and encodes to zero;
//  * the sign of x is put back (a -0 input would otherwise come out +0).
// Checked against the IEEE division for every BF16 input at 30,000 scales
// (host FMA), and on the GPU against the oracle by the exhaustive quantize
// tests.
__device__ __forceinline__ float div_by_scale(float x, float s, float r, float lim) {
  const float xc = __builtin_elementwise_minimum(__builtin_elementwise_maximum(x, -lim), lim);
  const float q0 = __fmul_rn(xc, r);
  const float e = __builtin_fmaf(-q0, s, xc);
  const float q1 = __builtin_fmaf(e, r, q0);
  return __builtin_copysignf(q1, xc);
}
__device__ __forceinline__ bool div_by_scale_ok(float s) {
  return s >= 0x1p-60f && s <= 0x1p60f;
}

// SiLU(g) * u in FP32: g * (1 / (1 + exp(-g))) * u, with the hardware
// exponential and reciprocal (about 1 ulp each).  For very negative g,
// exp(-g) overflows to +Inf, its reciprocal is 0 and the result is a zero
// with the sign of g * u, as in exact arithmetic.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __expf(-g);
  const float s = __fmul_rn(g, __builtin_amdgcn_rcpf(__fadd_rn(1.0f, e)));
  return __fmul_rn(s, u);
}

// The SwiGLU variant of the pull request "Load static FP8 Cosmos3 Nano/Super
// checkpoints without re-quantizing them" (commit message on swiglu_alpha /
// swiglu_beta): alpha is a gain inside the sigmoid, beta an offset on up,
// g * sigmoid(alpha * g) * (u + beta).  A zero beta leaves u untouched (so a
// -0 stays -0) and 1 * g == g exactly, so (alpha, beta) = (1, 0) gives the
// bits of silu_mul.
__device__ __forceinline__ float silu_mul_ab(float g, float u, float alpha, float beta) {
  const float e = __expf(-__fmul_rn(alpha, g));
  const float s = __fmul_rn(g, __builtin_amdgcn_rcpf(__fadd_rn(1.0f, e)));
  return __fmul_rn(s, beta == 0.0f ? u : __fadd_rn(u, beta));
}

}  // namespace fp8mot
