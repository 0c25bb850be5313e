// HBM-bound kernels of libfp8mot: static activation quantization, two-input
// SwiGLU with FP8 output, and the amax observer.
//
// All three stream flat contiguous buffers: each thread handles 16 elements
// per step (two 128-bit BF16 loads per input, one 128-bit store of 16 FP8
// codes), the grid strides over 16-element units, and the last n % 16
// elements are done one by one by the first threads of block 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace fp8mot {

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Static quantization: q = e4m3(x / s), one IEEE FP32 division per element.
__global__ __launch_bounds__(kThreads) void quant_static_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, int64_t n,
    const float* __restrict__ d_scale) {
  const float s = *d_scale;
  const int64_t units = n >> 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x4* qv = reinterpret_cast<u32x4*>(q);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < units;
       i += stride) {
    const u32x4 a = __builtin_nontemporal_load(xv + 2 * i);
    const u32x4 b = __builtin_nontemporal_load(xv + 2 * i + 1);
    float f[16];
    unpack8(a, f);
    unpack8(b, f + 8);
    float qf[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) qf[j] = f[j] / s;   // IEEE division
    u32x4 o;
    o.x = e4m3_pack4(qf[0], qf[1], qf[2], qf[3]);
    o.y = e4m3_pack4(qf[4], qf[5], qf[6], qf[7]);
    o.z = e4m3_pack4(qf[8], qf[9], qf[10], qf[11]);
    o.w = e4m3_pack4(qf[12], qf[13], qf[14], qf[15]);
    __builtin_nontemporal_store(o, qv + i);
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 4) + threadIdx.x;
    if (t < n) q[t] = (uint8_t)e4m3_encode(bf16_to_f32(x[t]) / s);
  }
}

// Two-input SwiGLU: q = e4m3(silu(g) * u / s_out), the division done as a
// multiplication by the (correctly rounded) reciprocal of s_out.
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
    uint8_t* __restrict__ q, int64_t n, const float* __restrict__ d_s) {
  const float rs = 1.0f / *d_s;
  const int64_t units = n >> 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4* gv = reinterpret_cast<const u32x4*>(g);
  const u32x4* uv = reinterpret_cast<const u32x4*>(u);
  u32x4* qv = reinterpret_cast<u32x4*>(q);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < units;
       i += stride) {
    const u32x4 g0 = __builtin_nontemporal_load(gv + 2 * i);
    const u32x4 g1 = __builtin_nontemporal_load(gv + 2 * i + 1);
    const u32x4 u0 = __builtin_nontemporal_load(uv + 2 * i);
    const u32x4 u1 = __builtin_nontemporal_load(uv + 2 * i + 1);
    float fg[16], fu[16];
    unpack8(g0, fg);
    unpack8(g1, fg + 8);
    unpack8(u0, fu);
    unpack8(u1, fu + 8);
    float h[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) h[j] = __fmul_rn(silu_mul(fg[j], fu[j]), rs);
    u32x4 o;
    o.x = e4m3_pack4(h[0], h[1], h[2], h[3]);
    o.y = e4m3_pack4(h[4], h[5], h[6], h[7]);
    o.z = e4m3_pack4(h[8], h[9], h[10], h[11]);
    o.w = e4m3_pack4(h[12], h[13], h[14], h[15]);
    __builtin_nontemporal_store(o, qv + i);
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 4) + threadIdx.x;
    if (t < n)
      q[t] = (uint8_t)e4m3_encode(__fmul_rn(silu_mul(bf16_to_f32(g[t]), bf16_to_f32(u[t])), rs));
  }
}

// Folds the finished amax into the state and clears the reduction slots.
__device__ void observer_fold(fp8mot_observer_state_dev* st, int mode, float c) {
  const float a = __uint_as_float(
      __hip_atomic_load(&st->pending, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  float m = st->m;
  if (st->count == 0) {
    m = a;
  } else if (mode == 0) {
    m = (a != a || m != m) ? __builtin_nanf("") : (a > m ? a : m);
  } else {
    const float d = __fsub_rn(a, m);
    const float p = __fmul_rn(c, d);
    m = __fadd_rn(m, p);
  }
  st->m = m;
  st->count = st->count + 1;
  st->pending = 0u;
  st->arrivals = 0u;
}

// Block-wide max of non-negative FP32 bit patterns (integer order == value
// order for non-negative floats; NaN patterns sort above +Inf) into the
// state's pending slot; the last block to arrive folds it into the state.
__device__ __forceinline__ void block_max_and_fold(uint32_t v, fp8mot_observer_state_dev* st,
                                                   int mode, float c) {
  __shared__ uint32_t red[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = m > red[w] ? m : red[w];
    // only blocks that can raise the running max touch the shared word, so
    // the atomics do not serialize on one address across the whole grid
    if (m > __hip_atomic_load(&st->pending, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(&st->pending, m);
    __threadfence();
    const uint32_t prev = atomicAdd(&st->arrivals, 1u);
    if (prev == gridDim.x - 1) {
      __threadfence();
      observer_fold(st, mode, c);
    }
  }
}

// amax over BF16: max of (bits & 0x7FFF) as integers is max |x| exactly.
__global__ __launch_bounds__(kThreads) void amax_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t n, fp8mot_observer_state_dev* st, int mode,
    float c) {
  const int64_t units = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < units;
       i += stride) {
    const u32x4 a = __builtin_nontemporal_load(xv + i);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
      m = m > lo ? m : lo;
      m = m > hi ? m : hi;
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 3) + threadIdx.x;
    if (t < n) {
      const uint32_t v = x[t] & 0x7FFFu;
      m = m > v ? m : v;
    }
  }
  block_max_and_fold(m << 16, st, mode, c);
}

// amax of silu(g) * u in FP32 (as silu_mul_kernel evaluates it).
__global__ __launch_bounds__(kThreads) void amax_swiglu_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ u, int64_t n,
    fp8mot_observer_state_dev* st, int mode, float c) {
  const int64_t units = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4* gv = reinterpret_cast<const u32x4*>(g);
  const u32x4* uv = reinterpret_cast<const u32x4*>(u);
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < units;
       i += stride) {
    float fg[8], fu[8];
    unpack8(__builtin_nontemporal_load(gv + i), fg);
    unpack8(__builtin_nontemporal_load(uv + i), fu);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = __float_as_uint(silu_mul(fg[j], fu[j])) & 0x7FFFFFFFu;
      m = m > v ? m : v;
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 3) + threadIdx.x;
    if (t < n) {
      const uint32_t v =
          __float_as_uint(silu_mul(bf16_to_f32(g[t]), bf16_to_f32(u[t]))) & 0x7FFFFFFFu;
      m = m > v ? m : v;
    }
  }
  block_max_and_fold(m, st, mode, c);
}

__global__ void scale_from_state_kernel(const fp8mot_observer_state_dev* st,
                                        float* scale) {
  *scale = st->m / 448.0f;
}

int grid_for(int64_t units, int max_blocks) {
  int64_t b = (units + kThreads - 1) / kThreads;
  if (b < 1) b = 1;
  if (b > max_blocks) b = max_blocks;
  return (int)b;
}

}  // namespace

hipError_t launch_quant_static(const uint16_t* x, uint8_t* q, int64_t n,
                               const float* d_scale, int max_blocks,
                               hipStream_t stream) {
  hipLaunchKernelGGL(quant_static_kernel, dim3(grid_for(n >> 4, max_blocks)),
                     dim3(kThreads), 0, stream, x, q, n, d_scale);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, uint8_t* q,
                           int64_t n, const float* d_s, int max_blocks,
                           hipStream_t stream) {
  hipLaunchKernelGGL(silu_mul_kernel, dim3(grid_for(n >> 4, max_blocks)),
                     dim3(kThreads), 0, stream, g, u, q, n, d_s);
  return hipGetLastError();
}

hipError_t launch_observe(const uint16_t* x, const uint16_t* u, int64_t n,
                          fp8mot_observer_state_dev* st, int mode, float c,
                          int max_blocks, hipStream_t stream) {
  // a reduction needs few blocks: two per CU, each striding over the input
  max_blocks = max_blocks / 4 > 0 ? max_blocks / 4 : 1;
  if (u == nullptr) {
    hipLaunchKernelGGL(amax_bf16_kernel, dim3(grid_for(n >> 3, max_blocks)),
                       dim3(kThreads), 0, stream, x, n, st, mode, c);
  } else {
    hipLaunchKernelGGL(amax_swiglu_kernel, dim3(grid_for(n >> 3, max_blocks)),
                       dim3(kThreads), 0, stream, x, u, n, st, mode, c);
  }
  return hipGetLastError();
}

hipError_t launch_scale_from_state(const fp8mot_observer_state_dev* st,
                                   float* scale, hipStream_t stream) {
  hipLaunchKernelGGL(scale_from_state_kernel, dim3(1), dim3(1), 0, stream, st,
                     scale);
  return hipGetLastError();
}

}  // namespace fp8mot
