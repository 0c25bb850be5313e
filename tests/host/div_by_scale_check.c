// Host check of the quantize kernels' division (div_by_scale in
// mlp_fp8_quant_amd/csrc/device_common.h, restated here with the C library's
// correctly rounded fmaf): for every BF16 x and scales s in [2^-60, 2^60],
// the clamped Markstein quotient must give the E4M3 code of the IEEE
// quotient x / s, and the same FP32 quotient wherever |x / s| lies in
// [2^-12, 1024] (the range in which E4M3 rounding boundaries lie).
// Usage: div_by_scale_check <number of scales>; exit status 1 on a mismatch.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float fast(float x, float s, float r, float lim) {
  float xc = x;
  if (!(xc != xc)) { if (xc < -lim) xc = -lim; if (xc > lim) xc = lim; }
  float q0 = xc * r;
  float e = fmaf(-q0, s, xc);
  float q1 = fmaf(e, r, q0);
  return copysignf(q1, xc);
}
// E4M3 code of v (RNE, saturating, NaN 0x7F, sign kept) -- integer version
static uint32_t enc(float v) {
  uint32_t u = u32(v), a = u & 0x7FFFFFFFu, code;
  if (a > 0x7F800000u) return 0x7F;
  if (a >= 0x43E00000u) code = 0x7E;
  else if (a >= 0x3C800000u) code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - 0x3C0u;
  else { float f = f32(a) + 16384.0f; code = u32(f) - 0x46800000u; }
  return code | ((u >> 24) & 0x80u);
}
int main(int argc, char** argv) {
  long nscales = argc > 1 ? atol(argv[1]) : 20000;
  uint64_t rng = 0x9E3779B97F4A7C15ull;
  long bad_q = 0, bad_code = 0, checked = 0;
  for (long t = 0; t < nscales; ++t) {
    float s;
    if (t < nscales / 3) {
      // scales next to "nice" values (k ulps away), as the GPU tests use
      const float base[] = {1.0f, 3.0f, 0.0123f, 0.02f, 0.1f, 1.337f, 20.0f / 448, 0.75f};
      float m = base[t % 8]; int k = (int)(t / 8) % 41 - 20;   // -20 .. 20 FP32 units away
      s = f32(u32(m) + k);
    } else {
      rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
      double e = ((rng >> 11) * (1.0 / 9007199254740992.0)) * 120.0 - 60.0;
      rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
      s = (float)ldexp(1.0 + (rng >> 11) * (1.0 / 9007199254740992.0), (int)floor(e));
    }
    if (!(s >= 0x1p-60f && s <= 0x1p60f)) continue;
    float r = 1.0f / s, lim = 1024.0f * s;
    for (uint32_t b = 0; b < 65536; ++b) {
      float x = f32(b << 16);
      float qi = x / s, qf = fast(x, s, r, lim);
      ++checked;
      if (enc(qi) != enc(qf)) {
        if (bad_code < 10) printf("code mismatch s=%a x=%a ieee=%a fast=%a\n", s, x, qi, qf);
        ++bad_code;
      }
      float aq = fabsf(qi);
      if (aq >= 0x1p-12f && aq <= 1024.0f && u32(qi) != u32(qf)) {
        if (bad_q < 10) printf("quotient mismatch s=%a x=%a ieee=%a fast=%a\n", s, x, qi, qf);
        ++bad_q;
      }
    }
  }
  printf("checked %ld, quotient mismatches %ld, code mismatches %ld\n", checked, bad_q, bad_code);
  return bad_code != 0;
}
