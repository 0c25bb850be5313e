// HBM-bound kernels of libfp8mot: static activation quantization, SwiGLU with
// FP8 output (two-input, and one-input with gate and up adjacent), and the
// amax observer.
//
// All three stream flat contiguous buffers with 128-bit nontemporal loads and
// stores, several in flight per thread; the grid strides over 16-element
// units and the last n % 16 elements are done one by one by the first
// threads of block 0.
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

// Static quantization: q = e4m3(x / s) with the IEEE FP32 quotient's codes
// (div_by_scale for scales in [2^-60, 2^60], the division itself otherwise).
// A thread handles 32 elements per step (four 128-bit loads in flight, two
// 128-bit stores) on a grid of up to 64 workgroups per CU, so that the
// large-MLP activation is one grid step (measured on MI355X at 84M elements:
// 43.9 us against 46-47 us with 64 elements per thread on half the grid, and
// against 43.2 us for a kernel with the same accesses and no arithmetic).
__global__ __launch_bounds__(kThreads) void quant_static_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, int64_t n,
    const float* __restrict__ d_scale) {
  const float s = *d_scale;
  const bool fast = div_by_scale_ok(s);         // uniform
  const float r = 1.0f / s, lim = 1024.0f * s;
  const int64_t units = n >> 4;                 // 16-element units
  constexpr int UN = 2;                         // units in flight per thread
  const int64_t stride = (int64_t)gridDim.x * kThreads * UN;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x4* qv = reinterpret_cast<u32x4*>(q);
  for (int64_t base = (int64_t)blockIdx.x * kThreads * UN + threadIdx.x; base < units;
       base += stride) {
    u32x4 a[UN][2];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        a[k][0] = __builtin_nontemporal_load(xv + 2 * i);
        a[k][1] = __builtin_nontemporal_load(xv + 2 * i + 1);
      }
    }
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        float f[16];
        unpack8(a[k][0], f);
        unpack8(a[k][1], f + 8);
        if (fast) {
#pragma unroll
          for (int j = 0; j < 16; ++j) f[j] = div_by_scale(f[j], s, r, lim);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) f[j] = f[j] / s;   // IEEE division
        }
        u32x4 o;
        o.x = e4m3_pack4(f[0], f[1], f[2], f[3]);
        o.y = e4m3_pack4(f[4], f[5], f[6], f[7]);
        o.z = e4m3_pack4(f[8], f[9], f[10], f[11]);
        o.w = e4m3_pack4(f[12], f[13], f[14], f[15]);
        __builtin_nontemporal_store(o, qv + i);
      }
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 4) + threadIdx.x;
    if (t < n) q[t] = (uint8_t)e4m3_encode(bf16_to_f32(x[t]) / s);
  }
}

// SwiGLU with FP8 output: q = e4m3(g * sigmoid(alpha g) * (u + beta) / s_out),
// the division done as a multiplication by the (correctly rounded)
// reciprocal of s_out.  A thread handles 64 elements per step: sixteen
// 128-bit loads in flight, four stores (measured on MI355X at the large-MLP
// size: 4 units per thread beat 1 and 2; the grid takes up to 64 workgroups
// per CU: 366 -> 355 us against 32, 372 us with 16).
//  ADJ = false: g and u are two flat tensors of n elements (two-input form).
//  ADJ = true:  one tensor x of rows [gate (I) | up (I)], I % 16 == 0; the
//               output is [rows, I] and n = rows * I.  Each 16-element unit
//               lies inside one row half.
template <bool ADJ>
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
    uint8_t* __restrict__ q, int64_t n, const float* __restrict__ d_s,
    float alpha, float beta, uint32_t inter) {
  const float rs = 1.0f / *d_s;
  const int64_t units = n >> 4;
  constexpr int UN = 4;                         // units in flight per thread
  const int64_t stride = (int64_t)gridDim.x * kThreads * UN;
  const uint32_t upr = inter >> 4;              // ADJ: units per row
  u32x4* qv = reinterpret_cast<u32x4*>(q);
  // element offset of unit i's gate values (its up values follow at +inter)
  auto gate_at = [&](int64_t i) -> int64_t {
    if constexpr (ADJ) {
      const uint32_t r = (uint32_t)i / upr, c = (uint32_t)i - r * upr;
      return (int64_t)r * (2 * (int64_t)inter) + 16 * (int64_t)c;
    } else {
      return 16 * i;
    }
  };
  for (int64_t base = (int64_t)blockIdx.x * kThreads * UN + threadIdx.x; base < units;
       base += stride) {
    u32x4 a[UN][4];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        const int64_t e = gate_at(i);
        const u32x4* gp = reinterpret_cast<const u32x4*>(g + e);
        const u32x4* up = reinterpret_cast<const u32x4*>(ADJ ? g + e + inter : u + e);
        a[k][0] = __builtin_nontemporal_load(gp);
        a[k][1] = __builtin_nontemporal_load(gp + 1);
        a[k][2] = __builtin_nontemporal_load(up);
        a[k][3] = __builtin_nontemporal_load(up + 1);
      }
    }
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        float fg[16], fu[16];
        unpack8(a[k][0], fg);
        unpack8(a[k][1], fg + 8);
        unpack8(a[k][2], fu);
        unpack8(a[k][3], fu + 8);
        float h[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) h[j] = __fmul_rn(silu_mul_ab(fg[j], fu[j], alpha, beta), rs);
        u32x4 o;
        o.x = e4m3_pack4(h[0], h[1], h[2], h[3]);
        o.y = e4m3_pack4(h[4], h[5], h[6], h[7]);
        o.z = e4m3_pack4(h[8], h[9], h[10], h[11]);
        o.w = e4m3_pack4(h[12], h[13], h[14], h[15]);
        __builtin_nontemporal_store(o, qv + i);
      }
    }
  }
  if (!ADJ && blockIdx.x == 0) {
    const int64_t t = (units << 4) + threadIdx.x;
    if (t < n)
      q[t] = (uint8_t)e4m3_encode(
          __fmul_rn(silu_mul_ab(bf16_to_f32(g[t]), bf16_to_f32(u[t]), alpha, beta), rs));
  }
}

// Read/write ceiling for the byte mix of the two HBM-bound kernels, with no
// arithmetic: NIN = 1 reads 2 bytes and writes 1 per element (quantize),
// NIN = 2 reads 2 + 2 and writes 1 (two-input SwiGLU).  Same loop, units in
// flight (UN), nontemporal 128-bit accesses and grid as quant_static_kernel /
// silu_mul_kernel; each output byte is the low byte of the XOR of its input
// words, so every load is used.  A measurement aid: the quantize and SwiGLU
// kernels are measured against what the memory system delivers for their mix
// (on MI355X these are also the fastest of the unit counts and grid sizes
// swept for a plain read/write stream of that mix).
template <int NIN, int UN>
__global__ __launch_bounds__(kThreads) void rw_ceiling_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    uint8_t* __restrict__ out, int64_t n) {
  const int64_t units = n >> 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads * UN;
  const u32x4* av = reinterpret_cast<const u32x4*>(a);
  const u32x4* bv = reinterpret_cast<const u32x4*>(b);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  for (int64_t base = (int64_t)blockIdx.x * kThreads * UN + threadIdx.x; base < units;
       base += stride) {
    u32x4 x[UN][2 * NIN];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        x[k][0] = __builtin_nontemporal_load(av + 2 * i);
        x[k][1] = __builtin_nontemporal_load(av + 2 * i + 1);
        if constexpr (NIN == 2) {
          x[k][2] = __builtin_nontemporal_load(bv + 2 * i);
          x[k][3] = __builtin_nontemporal_load(bv + 2 * i + 1);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        u32x4 lo = x[k][0], hi = x[k][1];
        if constexpr (NIN == 2) {
          lo ^= x[k][2];
          hi ^= x[k][3];
        }
        // byte j of the output: low byte of input word j
        auto pick = [](uint32_t w0, uint32_t w1) {
          return (w0 & 0xFFu) | ((w0 >> 8) & 0xFF00u) | ((w1 & 0xFFu) << 16) | ((w1 << 8) & 0xFF000000u);
        };
        u32x4 o;
        o.x = pick(lo.x, lo.y);
        o.y = pick(lo.z, lo.w);
        o.z = pick(hi.x, hi.y);
        o.w = pick(hi.z, hi.w);
        __builtin_nontemporal_store(o, ov + i);
      }
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 4) + threadIdx.x;
    if (t < n) out[t] = (uint8_t)(NIN == 2 ? a[t] ^ b[t] : a[t]);
  }
}

// One-input SwiGLU for rows whose width I is not a multiple of 16: one
// element per thread per step (such rows are not 16-byte aligned).
__global__ __launch_bounds__(kThreads) void silu_mul_adj_scalar_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, int64_t n,
    const float* __restrict__ d_s, float alpha, float beta, int64_t inter) {
  const float rs = 1.0f / *d_s;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t r = e / inter, c = e - r * inter;
    const uint16_t* row = x + r * 2 * inter;
    q[e] = (uint8_t)e4m3_encode(
        __fmul_rn(silu_mul_ab(bf16_to_f32(row[c]), bf16_to_f32(row[inter + c]), alpha, beta), rs));
  }
}

// Per-token (per-row) dynamic quantization (model card "Cosmos3-Nano-Policy-
// DROID, FP8 + RTN + moving-average activation observer", section 3.2:
// per-channel weights, per-token activations).  One workgroup per row of K
// elements (K % 16 == 0).  The row's amax is the integer max of
// (bits & 0x7FFF) -- exact, and NaN patterns sort above Inf; scale =
// fp32(amax) / 448; q = e4m3(x / s) with the IEEE quotient's codes
// (div_by_scale when the row's scale is in its range).  A
// zero row (s = 0) keeps its signed zeros; a NaN row gets a NaN scale and
// all-NaN codes.  UH > 0: the row stays in registers between the amax and
// the quantization (up to UH 16-element units per thread); UH == 0: the row
// is read twice (the second time from cache).
template <int UH>
__global__ __launch_bounds__(kThreads) void quant_per_row_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
    float* __restrict__ scales, int64_t rows, int64_t K) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t units = K >> 4;                 // 16-element units per row
  auto max16 = [](uint32_t m, const u32x4 a, const u32x4 b) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
      m = m > lo ? m : lo;
      m = m > hi ? m : hi;
    }
    return m;
  };
  auto encode16 = [](const u32x4 a, const u32x4 b, float s) {
    float f[16];
    unpack8(a, f);
    unpack8(b, f + 8);
    if (div_by_scale_ok(s)) {                          // uniform per row
      const float r = 1.0f / s, lim = 1024.0f * s;
#pragma unroll
      for (int j = 0; j < 16; ++j) f[j] = div_by_scale(f[j], s, r, lim);
    } else if (s != 0.0f) {
#pragma unroll
      for (int j = 0; j < 16; ++j) f[j] = f[j] / s;   // IEEE division
    }
    u32x4 o;
    o.x = e4m3_pack4(f[0], f[1], f[2], f[3]);
    o.y = e4m3_pack4(f[4], f[5], f[6], f[7]);
    o.z = e4m3_pack4(f[8], f[9], f[10], f[11]);
    o.w = e4m3_pack4(f[12], f[13], f[14], f[15]);
    return o;
  };
  // UH > 0: the next row's loads are issued before this row is reduced and
  // encoded, so one row's memory round trip overlaps another's arithmetic
  u32x4 hold[UH > 0 ? UH : 1][2], next[UH > 0 ? UH : 1][2];
  auto load_row = [&](u32x4 (*dst)[2], int64_t r) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + r * K);
#pragma unroll
    for (int k = 0; k < UH; ++k) {
      const int64_t i = threadIdx.x + k * kThreads;
      if (i < units) {
        dst[k][0] = __builtin_nontemporal_load(xr + 2 * i);
        dst[k][1] = __builtin_nontemporal_load(xr + 2 * i + 1);
      }
    }
  };
  if constexpr (UH > 0) {
    if (blockIdx.x < rows) load_row(next, blockIdx.x);
  }
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + r * K);
    u32x4* qr = reinterpret_cast<u32x4*>(q + r * K);
    uint32_t m = 0;
    if constexpr (UH > 0) {
#pragma unroll
      for (int k = 0; k < UH; ++k) {
        hold[k][0] = next[k][0];
        hold[k][1] = next[k][1];
      }
      if (r + gridDim.x < rows) load_row(next, r + gridDim.x);
#pragma unroll
      for (int k = 0; k < UH; ++k)
        if (threadIdx.x + k * kThreads < units) m = max16(m, hold[k][0], hold[k][1]);
    } else {
      for (int64_t i = threadIdx.x; i < units; i += kThreads) m = max16(m, xr[2 * i], xr[2 * i + 1]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = __shfl_xor(m, off, 64);
      m = m > o ? m : o;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) m = m > red[w] ? m : red[w];
    const float s = __uint_as_float(m << 16) / 448.0f;
    if (threadIdx.x == 0) scales[r] = s;
    if constexpr (UH > 0) {
#pragma unroll
      for (int k = 0; k < UH; ++k) {
        const int64_t i = threadIdx.x + k * kThreads;
        if (i < units) __builtin_nontemporal_store(encode16(hold[k][0], hold[k][1], s), qr + i);
      }
    } else {
      for (int64_t i = threadIdx.x; i < units; i += kThreads)
        qr[i] = encode16(xr[2 * i], xr[2 * i + 1], s);
    }
    __syncthreads();   // red is reused by the next row
  }
}

// Re-quantization onto the group's largest scale: what a fused projection
// that keeps one scale does to each member (pull request "Load static FP8
// Cosmos3 Nano/Super checkpoints without re-quantizing them", "Description":
// FP8-round((s_i * qW_i) / max(s)) instead of keeping s_i * qW_i).  Kept to
// build the fused-topology comparison; the split path never calls it.
// out = e4m3(fp32(fp32(s_i * dec(q)) / s_max)), decode by the hardware FP8 ->
// FP32 conversion (exact; NaN codes give NaN).  16 codes per thread per step.
__global__ __launch_bounds__(kThreads) void requant_onto_max_kernel(
    const uint8_t* __restrict__ q, uint8_t* __restrict__ out, int64_t n,
    const float* __restrict__ s_i, const float* __restrict__ s_group, int group) {
  const float si = *s_i;
  float smax = s_group[0];
  for (int k = 1; k < group; ++k) smax = smax > s_group[k] ? smax : s_group[k];
  const int64_t units = n >> 4;
  const u32x4* qv = reinterpret_cast<const u32x4*>(q);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  auto requant4 = [&](uint32_t w) -> uint32_t {
    float f[4];
    f[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    f[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    f[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    f[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __fmul_rn(si, f[j]) / smax;
    return e4m3_pack4(f[0], f[1], f[2], f[3]);
  };
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < units;
       i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = qv[i];
    u32x4 o;
    o.x = requant4(v.x);
    o.y = requant4(v.y);
    o.z = requant4(v.z);
    o.w = requant4(v.w);
    ov[i] = o;
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 4) + threadIdx.x;
    if (t < n) out[t] = (uint8_t)(requant4(q[t]) & 0xFFu);
  }
}

// Block-wide max of non-negative FP32 bit patterns (integer order == value
// order for non-negative floats; NaN patterns sort above +Inf) into the
// state's pending slot.  Only a block that can raise the running value
// issues the atomic, so the atomics do not serialize on one address.
__device__ __forceinline__ void block_max_to(uint32_t v, uint32_t* dst) {
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
    if (m > __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(dst, m);
  }
}

// Folds the call's amax (st->pending) into the state and clears the slot:
// the first call sets m, later calls take the max (NaN sticks) or the moving
// average m + c * (a - m) in three separately rounded FP32 operations.
__device__ __forceinline__ void observer_fold(fp8mot_observer_state_dev* st, int mode, float c) {
  const float a = __uint_as_float(
      __hip_atomic_load(&st->pending, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  float m = st->m;
  const int32_t count = st->count;
  if (count == 0) {
    m = a;
  } else if (mode == 0) {
    m = (a != a || m != m) ? __builtin_nanf("") : (a > m ? a : m);
  } else {
    const float d = __fsub_rn(a, m);
    const float p = __fmul_rn(c, d);
    m = __fadd_rn(m, p);
  }
  st->m = m;
  st->count = count + 1;
  st->pending = 0u;
  st->arrived = 0u;
}

// End of an amax workgroup when the fold happens in the same launch: after
// its atomic max, each workgroup counts itself in (release); the last one to
// arrive (acquire) sees every workgroup's max and folds it into the state.
__device__ __forceinline__ void arrive_and_fold(fp8mot_observer_state_dev* st, int mode, float c) {
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t prev = atomicAdd(&st->arrived, 1u);
    if (prev == gridDim.x - 1) {
      __threadfence();
      observer_fold(st, mode, c);
    }
  }
}

// amax over BF16: max of (bits & 0x7FFF) as integers is max |x| exactly.
// Sixteen 128-bit loads in flight per thread per step, so that a workgroup's
// 32K-element share is one memory round trip rather than four.  When the
// grid is capped and every workgroup walks several shares (LOOP), eight
// loads per step with the next step's loads issued before this step's
// reduction keep the memory busy instead (84M elements 28.9 -> 26.2 us; for
// a single share the one round trip is faster: 4M elements 7.4 against 8.6).
template <bool LOOP>
__global__ __launch_bounds__(kThreads) void amax_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t n, fp8mot_observer_state_dev* st, int mode, float c,
    int fold) {
  uint32_t* pending = &st->pending;
  const int64_t units = n >> 3;                 // 8-element units
  constexpr int UN = LOOP ? 8 : 16;             // units per thread per step
  const int64_t stride = (int64_t)gridDim.x * kThreads * UN;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  uint32_t m = 0;
  auto load = [&](u32x4* d, int64_t base) {
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t i = base + k * kThreads;
      d[k] = i < units ? __builtin_nontemporal_load(xv + i) : (u32x4){0, 0, 0, 0};
    }
  };
  auto reduce = [&](const u32x4* a) {
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const uint32_t w[4] = {a[k].x, a[k].y, a[k].z, a[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
      }
    }
  };
  int64_t base = (int64_t)blockIdx.x * kThreads * UN + threadIdx.x;
  u32x4 a[UN];
  if constexpr (LOOP) {
    u32x4 nx[UN];
    if (base < units) load(nx, base);
    for (; base < units; base += stride) {
#pragma unroll
      for (int k = 0; k < UN; ++k) a[k] = nx[k];
      if (base + stride < units) load(nx, base + stride);
      reduce(a);
    }
  } else {
    for (; base < units; base += stride) {
      load(a, base);
      reduce(a);
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t = (units << 3) + threadIdx.x;
    if (t < n) {
      const uint32_t v = x[t] & 0x7FFFu;
      m = m > v ? m : v;
    }
  }
  block_max_to(m << 16, pending);
  if (fold) arrive_and_fold(st, mode, c);
}

// amax of silu(g) * u in FP32 (as silu_mul_kernel evaluates it).  Four
// 8-element units per thread per step.
__global__ __launch_bounds__(kThreads) void amax_swiglu_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ u, int64_t n,
    fp8mot_observer_state_dev* st, int mode, float c, int fold) {
  uint32_t* pending = &st->pending;
  const int64_t units = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kThreads * 4;
  const u32x4* gv = reinterpret_cast<const u32x4*>(g);
  const u32x4* uv = reinterpret_cast<const u32x4*>(u);
  uint32_t m = 0;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * 4 + threadIdx.x; base < units;
       base += stride) {
    u32x4 a[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t i = base + k * kThreads;
      if (i < units) {
        a[k][0] = __builtin_nontemporal_load(gv + i);
        a[k][1] = __builtin_nontemporal_load(uv + i);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (base + k * kThreads < units) {
        float fg[8], fu[8];
        unpack8(a[k][0], fg);
        unpack8(a[k][1], fu);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t v = __float_as_uint(silu_mul(fg[j], fu[j])) & 0x7FFFFFFFu;
          m = m > v ? m : v;
        }
      }
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
  block_max_to(m, pending);
  if (fold) arrive_and_fold(st, mode, c);
}

// Folds the pending amax into the state and clears the slot.  One thread.
__global__ void observer_update_kernel(fp8mot_observer_state_dev* st, int mode,
                                       float c) {
  observer_fold(st, mode, c);
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

// Grids of the two streaming kernels (max_blocks = 8 per CU): one thread per
// 32 (quantize) or 64 (SwiGLU) elements, up to 64 workgroups per CU.
static int quant_grid(int64_t n, int max_blocks) { return grid_for(n >> 5, 8 * max_blocks); }
static int silu_grid(int64_t n, int max_blocks) { return grid_for(n >> 6, 8 * max_blocks); }

hipError_t launch_quant_static(const uint16_t* x, uint8_t* q, int64_t n,
                               const float* d_scale, int max_blocks,
                               hipStream_t stream) {
  hipLaunchKernelGGL(quant_static_kernel, dim3(quant_grid(n, max_blocks)),
                     dim3(kThreads), 0, stream, x, q, n, d_scale);
  return hipGetLastError();
}

hipError_t launch_quant_per_row(const uint16_t* x, uint8_t* q, float* scales,
                                int64_t rows, int64_t K, int max_blocks,
                                hipStream_t stream) {
  const int64_t b = rows < 2 * (int64_t)max_blocks ? rows : 2 * (int64_t)max_blocks;
  const dim3 grid((unsigned)(b > 0 ? b : 1)), block(kThreads);
  const int64_t units = K >> 4;
  // keep the row in registers when it fits 2 or 8 units per thread
  if (units <= 2 * kThreads)
    hipLaunchKernelGGL(quant_per_row_kernel<2>, grid, block, 0, stream, x, q, scales, rows, K);
  else if (units <= 8 * kThreads)
    hipLaunchKernelGGL(quant_per_row_kernel<8>, grid, block, 0, stream, x, q, scales, rows, K);
  else
    hipLaunchKernelGGL(quant_per_row_kernel<0>, grid, block, 0, stream, x, q, scales, rows, K);
  return hipGetLastError();
}

hipError_t launch_requant_onto_max(const uint8_t* q, uint8_t* out, int64_t n,
                                   const float* s_i, const float* s_group, int group,
                                   int max_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(requant_onto_max_kernel, dim3(grid_for(n >> 4, max_blocks)),
                     dim3(kThreads), 0, stream, q, out, n, s_i, s_group, group);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, uint8_t* q,
                           int64_t n, const float* d_s, float alpha, float beta,
                           int max_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(silu_mul_kernel<false>, dim3(silu_grid(n, max_blocks)),
                     dim3(kThreads), 0, stream, g, u, q, n, d_s, alpha, beta, 0u);
  return hipGetLastError();
}

hipError_t launch_rw_ceiling(const uint16_t* a, const uint16_t* b, uint8_t* out, int64_t n,
                             int max_blocks, hipStream_t stream) {
  if (b == nullptr)
    hipLaunchKernelGGL((rw_ceiling_kernel<1, 2>), dim3(quant_grid(n, max_blocks)),
                       dim3(kThreads), 0, stream, a, b, out, n);
  else
    hipLaunchKernelGGL((rw_ceiling_kernel<2, 4>), dim3(silu_grid(n, max_blocks)),
                       dim3(kThreads), 0, stream, a, b, out, n);
  return hipGetLastError();
}

hipError_t launch_silu_mul_adjacent(const uint16_t* x, uint8_t* q, int64_t rows,
                                    int64_t inter, const float* d_s, float alpha,
                                    float beta, int max_blocks, hipStream_t stream) {
  const int64_t n = rows * inter;
  if (inter % 16 == 0 && n / 16 <= (int64_t)UINT32_MAX) {
    hipLaunchKernelGGL(silu_mul_kernel<true>, dim3(silu_grid(n, max_blocks)),
                       dim3(kThreads), 0, stream, x, nullptr, q, n, d_s, alpha, beta,
                       (uint32_t)inter);
  } else {
    hipLaunchKernelGGL(silu_mul_adj_scalar_kernel, dim3(grid_for(n, 4 * max_blocks)),
                       dim3(kThreads), 0, stream, x, q, n, d_s, alpha, beta, inter);
  }
  return hipGetLastError();
}

hipError_t launch_observe(const uint16_t* x, const uint16_t* u, int64_t n,
                          fp8mot_observer_state_dev* st, int mode, float c,
                          int max_blocks, hipStream_t stream) {
  // Every workgroup ends in (at most) one atomic on the same word, and those
  // serialize: keep the grid at about one workgroup per 32K elements, and at
  // most two per CU (measured on MI355X: for 4M elements 128 workgroups take
  // 6.2 us and 512 take 8.6; for 52M, 512 take 17.8 us and 256 take 23.8).
  // With sixteen loads in flight per thread a workgroup's share is one memory
  // round trip: 4M elements 7.0 -> 4.1 us, 84M elements 26.8 us (6.3 TB/s).
  const int64_t want = (n + 32767) / 32768;
  const int cap = max_blocks / 4 > 0 ? max_blocks / 4 : 1;
  const int amax_blocks = want < 1 ? 1 : (want < cap ? (int)want : cap);
  // Small grids fold the call's amax into the state in the last workgroup
  // to finish; large ones in a second one-thread launch.  Each workgroup's
  // release fence before its arrival count writes back its XCD's L2 (the 8
  // XCDs' L2s are not coherent with one another), which is cheaper than a
  // second launch for up to 128 workgroups (4M elements: 10.4 -> 7.6 us per
  // call) and far dearer for 512 (84M elements: 28.5 -> 54.3 us).
  const int64_t blocks = u == nullptr ? grid_for(n >> 7, amax_blocks) : grid_for(n >> 5, amax_blocks);
  const int fold = blocks <= 128;
  if (u == nullptr) {
    if (want > amax_blocks)   // capped grid: every workgroup walks several shares
      hipLaunchKernelGGL(amax_bf16_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                         stream, x, n, st, mode, c, fold);
    else
      hipLaunchKernelGGL(amax_bf16_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                         stream, x, n, st, mode, c, fold);
  } else {
    hipLaunchKernelGGL(amax_swiglu_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       x, u, n, st, mode, c, fold);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fold) return e;
  hipLaunchKernelGGL(observer_update_kernel, dim3(1), dim3(1), 0, stream, st, mode, c);
  return hipGetLastError();
}

hipError_t launch_scale_from_state(const fp8mot_observer_state_dev* st,
                                   float* scale, hipStream_t stream) {
  hipLaunchKernelGGL(scale_from_state_kernel, dim3(1), dim3(1), 0, stream, st,
                     scale);
  return hipGetLastError();
}

}  // namespace fp8mot
