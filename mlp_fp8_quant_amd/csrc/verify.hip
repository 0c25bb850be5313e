// Verification aid, not a step of the path: the kernels' own FP32 -> E4M3
// and FP32 -> BF16 conversions applied to caller-given FP32 values, so that
// a test can run them over every FP32 bit pattern.  Each kind calls the
// device_common.h helper that the path's kernels call:
//   kind 0: e4m3_pack4, the packed conversion of the quantize and SwiGLU
//           kernels' vector bodies and of the GEMMs' FP8 output;
//   kind 1: e4m3_encode, the integer encoder of the elementwise tails;
//   kind 2: bf16x2_rne, the packed BF16 conversion of the GEMM epilogues.
// Four inputs per thread and step: one 16-byte load, then one 4-byte (E4M3)
// or 8-byte (BF16) store, in a grid-stride loop over n / 4 groups.

#include "device_common.h"
#include "kernels.h"

namespace fp8mot {
namespace {

constexpr int kBlock = 256;

template <int KIND>
__global__ __launch_bounds__(kBlock) void convert_f32_kernel(const float4* __restrict__ x,
                                                             void* __restrict__ out,
                                                             int64_t groups) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x; g < groups; g += stride) {
    const float4 v = x[g];
    if constexpr (KIND == 0) {
      static_cast<uint32_t*>(out)[g] = e4m3_pack4(v.x, v.y, v.z, v.w);
    } else if constexpr (KIND == 1) {
      static_cast<uint32_t*>(out)[g] = e4m3_encode(v.x) | e4m3_encode(v.y) << 8 |
                                       e4m3_encode(v.z) << 16 | e4m3_encode(v.w) << 24;
    } else {
      static_cast<uint2*>(out)[g] = make_uint2(bf16x2_rne(v.x, v.y), bf16x2_rne(v.z, v.w));
    }
  }
}

}  // namespace

hipError_t launch_convert_f32(const float* x, void* out, int64_t n, int kind, int max_blocks,
                              hipStream_t stream) {
  const int64_t groups = n / 4;
  if (groups == 0) return hipSuccess;
  const int64_t want = (groups + kBlock - 1) / kBlock;
  const int blocks = (int)(want < max_blocks ? want : max_blocks);
  const float4* x4 = reinterpret_cast<const float4*>(x);
  switch (kind) {
    case 0: convert_f32_kernel<0><<<blocks, kBlock, 0, stream>>>(x4, out, groups); break;
    case 1: convert_f32_kernel<1><<<blocks, kBlock, 0, stream>>>(x4, out, groups); break;
    default: convert_f32_kernel<2><<<blocks, kBlock, 0, stream>>>(x4, out, groups); break;
  }
  return hipGetLastError();
}

}  // namespace fp8mot
