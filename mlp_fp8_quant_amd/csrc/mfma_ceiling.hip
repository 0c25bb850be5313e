// Measurement aid, not a step of the path: the rate the matrix cores sustain
// on given FP8 operand data with nothing else in the loop -- no stage copies,
// no LDS, no decodes, no epilogue.  The GEMM kernels are measured against it:
// under MI355X's power limit the GFX clock, and with it the MFMA rate, depends
// on how much the operand bits toggle, so the published dense peaks (2.5
// PFLOP/s F16, 5.0 FP8, at 2.4 GHz) are not what a run on Gaussian-like data
// can reach.
//
// Every wave builds four A and four B fragments from the caller's code
// buffers (each lane its own codes, indices wrapped into the buffers), then
// issues 8 * iters MFMAs on four independent accumulators, pairing the
// fragments in two rotations so that consecutive MFMAs see different data:
//   ENGINE 0: v_mfma_f32_32x32x16_f16 on the codes decoded exactly to F16
//             (the exact engine's instruction);
//   ENGINE 1: v_mfma_scale_f32_32x32x64_f8f6f4 on the raw E4M3 codes (the
//             native FP8 instruction, unit scales).

#include "kernels.h"

namespace fp8mot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// One workgroup of 8 waves per CU (two per SIMD), the occupancy of the GEMM's
// 256x256 tiles; four independent accumulators per wave keep the pipe issuing.
constexpr int kBlock = 512;
constexpr int kPerCu = 1;

// Four consecutive codes from p[start + j .. start + j + 3], indices wrapped
// into [0, n): start < n and j + 3 < 32 <= n, so one subtraction suffices.
__device__ __forceinline__ int load4(const uint8_t* __restrict__ p, int64_t n, int64_t start,
                                     int j) {
  uint32_t w = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int64_t i = start + j + t;
    i = i >= n ? i - n : i;
    w |= (uint32_t)p[i] << (8 * t);
  }
  return (int)w;
}

template <bool HIGH>
__device__ __forceinline__ int f16x2_of(int x) {
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HIGH));
}

template <int ENGINE>
__global__ __launch_bounds__(kBlock, 2) void mfma_ceiling_kernel(
    const uint8_t* __restrict__ a, int64_t na, const uint8_t* __restrict__ b, int64_t nb,
    int64_t iters, float* __restrict__ sink) {
  const int64_t lane = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  constexpr int kCodes = ENGINE == 0 ? 8 : 32;   // codes per lane per operand
  typedef typename std::conditional<ENGINE == 0, f16x8, v8i>::type frag_t;
  frag_t fa[4], fb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t ia = ((lane * 4 + s) * kCodes) % na;
    const int64_t ib = ((lane * 4 + s) * kCodes + 7919 * kCodes) % nb;   // B away from A
    if constexpr (ENGINE == 0) {
      const int a0 = load4(a, na, ia, 0), a1 = load4(a, na, ia, 4);
      const int b0 = load4(b, nb, ib, 0), b1 = load4(b, nb, ib, 4);
      fa[s] = __builtin_bit_cast(f16x8, (v4i){f16x2_of<false>(a0), f16x2_of<true>(a0),
                                              f16x2_of<false>(a1), f16x2_of<true>(a1)});
      fb[s] = __builtin_bit_cast(f16x8, (v4i){f16x2_of<false>(b0), f16x2_of<true>(b0),
                                              f16x2_of<false>(b1), f16x2_of<true>(b1)});
    } else {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        fa[s][w] = load4(a, na, ia, 4 * w);
        fb[s][w] = load4(b, nb, ib, 4 * w);
      }
    }
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  auto mfma = [](const frag_t& x, const frag_t& y, const v16f& c) {
    if constexpr (ENGINE == 0)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
  };
  for (int64_t it = 0; it < iters; ++it) {
    c0 = mfma(fa[0], fb[0], c0);
    c1 = mfma(fa[1], fb[1], c1);
    c2 = mfma(fa[2], fb[2], c2);
    c3 = mfma(fa[3], fb[3], c3);
    c0 = mfma(fa[1], fb[2], c0);
    c1 = mfma(fa[2], fb[3], c1);
    c2 = mfma(fa[3], fb[0], c2);
    c3 = mfma(fa[0], fb[1], c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  // Every lane's products feed this test, so none can be dropped; finite
  // E4M3 data never sums to this exact value.
  if (s == 0x1.5p-120f) sink[0] = s;
}

}  // namespace

int mfma_ceiling_grid(int num_cus) { return kPerCu * num_cus; }

double mfma_ceiling_flops(int num_cus, int64_t iters, int engine) {
  const double waves = (double)mfma_ceiling_grid(num_cus) * (kBlock / 64);
  const double per_mfma = 2.0 * 32 * 32 * (engine == 0 ? 16 : 64);
  return waves * 8.0 * (double)iters * per_mfma;
}

hipError_t launch_mfma_ceiling(const uint8_t* a, int64_t na, const uint8_t* b, int64_t nb,
                               int64_t iters, int engine, float* sink, int num_cus,
                               hipStream_t stream) {
  const dim3 grid((unsigned)mfma_ceiling_grid(num_cus));
  if (engine == 1)
    hipLaunchKernelGGL(mfma_ceiling_kernel<1>, grid, dim3(kBlock), 0, stream, a, na, b, nb,
                       iters, sink);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<0>, grid, dim3(kBlock), 0, stream, a, na, b, nb,
                       iters, sink);
  return hipGetLastError();
}

}  // namespace fp8mot
