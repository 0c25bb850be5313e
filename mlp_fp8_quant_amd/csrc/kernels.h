// Internal launcher interface between the C ABI (capi.hip) and the kernels.
// Launchers assume validated arguments: non-negative sizes, 16-byte aligned
// pointers, K % 16 == 0, non-null scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mot {

// Device layout of fp8mot_observer_state (include/fp8mot.h).
struct fp8mot_observer_state_dev {
  float m;
  int32_t count;
  uint32_t pending;   // FP32 bit pattern of the running amax of the current call
  uint32_t arrived;   // workgroups of the current call that have added their max
};

hipError_t launch_quant_static(const uint16_t* x, uint8_t* q, int64_t n,
                               const float* d_scale, int max_blocks,
                               hipStream_t stream);

// Per-row dynamic quantization of x [rows, K] (K % 16 == 0): scales[r] =
// amax(row r) / 448, q[r, :] = e4m3(x[r, :] / scales[r]).
hipError_t launch_quant_per_row(const uint16_t* x, uint8_t* q, float* scales,
                                int64_t rows, int64_t K, int max_blocks,
                                hipStream_t stream);

// q = e4m3(g * sigmoid(alpha g) * (u + beta) / s); (1, 0) is plain SwiGLU.
hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, uint8_t* q,
                           int64_t n, const float* d_s, float alpha, float beta,
                           int max_blocks, hipStream_t stream);

// The same from one tensor x of rows [gate (inter) | up (inter)] into
// q [rows, inter].
hipError_t launch_silu_mul_adjacent(const uint16_t* x, uint8_t* q, int64_t rows,
                                    int64_t inter, const float* d_s, float alpha,
                                    float beta, int max_blocks, hipStream_t stream);

// Measurement aid: reads a [n] (and b [n] when not NULL) as 16-bit words and
// writes out [n] bytes, with the access pattern and grid of the quantize
// (b NULL) or two-input SwiGLU kernel and no arithmetic.
hipError_t launch_rw_ceiling(const uint16_t* a, const uint16_t* b, uint8_t* out, int64_t n,
                             int max_blocks, hipStream_t stream);

// Measurement aid: dense MFMAs on fragments built from the code buffers a [na]
// and b [nb] (na, nb >= 64; indices wrapped), 8 * iters per wave, engine 0 F16 on decoded
// codes, 1 native FP8; mfma_ceiling_grid(num_cus) workgroups of 512 threads (one per CU).
// sink: one float, written only if the products sum to a sentinel.
int mfma_ceiling_grid(int num_cus);
double mfma_ceiling_flops(int num_cus, int64_t iters, int engine);
hipError_t launch_mfma_ceiling(const uint8_t* a, int64_t na, const uint8_t* b, int64_t nb,
                               int64_t iters, int engine, float* sink, int num_cus,
                               hipStream_t stream);

// Verification aid: out = the kernels' conversion of x [n] (n % 4 == 0, both
// 16-byte aligned): kind 0 e4m3_pack4 and kind 1 e4m3_encode into n bytes,
// kind 2 bf16x2_rne into n 16-bit words.
hipError_t launch_convert_f32(const float* x, void* out, int64_t n, int kind, int max_blocks,
                              hipStream_t stream);

// u == nullptr: amax of the BF16 tensor x; otherwise amax of silu(x) * u.
hipError_t launch_observe(const uint16_t* x, const uint16_t* u, int64_t n,
                          fp8mot_observer_state_dev* st, int mode, float c,
                          int max_blocks, hipStream_t stream);

hipError_t launch_scale_from_state(const fp8mot_observer_state_dev* st,
                                   float* scale, hipStream_t stream);

// FP8 GEMM y[M,N] = (qa[M,K] . qb[N,K]^T) * (sx*sw), out_kind per fp8mot_out,
// accum per fp8mot_acc (0: F16 MFMA on exactly decoded codes, 1: FP8 MFMA).
// out_kind 3 (BF16) and 4 (FP32): sx [M] and sw [N] are per-row scales and
// y[m,n] = acc * fp32(sx[m] * sw[n]).
// ldc: row stride of y in elements (0: N, a contiguous y).
hipError_t launch_gemm(const uint8_t* qa, const uint8_t* qb, void* y,
                       int64_t M, int64_t N, int64_t K, const float* sx,
                       const float* sw, int out_kind, const float* sy,
                       int accum, int num_cus, hipStream_t stream, int64_t ldc = 0);

// True when launch_gemm of this shape and accumulation engine splits K over
// two wave groups of one workgroup: the sums of the even and of the odd 128-K
// stages are added at the end instead of one running sum over K.  That
// happens for 128x128 tiles (either engine) or 128x64 tiles (exact engine)
// with at most one tile per CU and K > N (a down projection short of tiles).
// Callers that promise bitwise equality between two launch shapes check it.
bool gemm_splits_k(int64_t M, int64_t N, int64_t K, int num_cus, int accum);

// Up to three BF16-output GEMMs of the same A in one launch (split Q/K/V):
// y[p] [M, N[p]] = (qa . qb[p]^T) * (sx * sw[p]); groups with N[p] == 0 must
// be left out by the caller.
hipError_t launch_gemm_grouped(const uint8_t* qa, int groups, const uint8_t* const* qb,
                               void* const* y, const int64_t* N, int64_t M, int64_t K,
                               const float* sx, const float* const* sw, int accum,
                               int num_cus, hipStream_t stream);

// Re-quantization of a fused group's member onto the group's largest scale
// (the failure mode of a single-scale fused group):
// out = e4m3(fp32(fp32(s_i * dec(q)) / max(s_group[0..group-1]))).
hipError_t launch_requant_onto_max(const uint8_t* q, uint8_t* out, int64_t n,
                                   const float* s_i, const float* s_group, int group,
                                   int max_blocks, hipStream_t stream);

// Gate and up GEMMs of a gated MLP with the SwiGLU-FP8 epilogue in one launch:
// qh[M,I] = e4m3(silu(bf16(G)) * bf16(U) / sh) with G = qx.wg^T * (sx*sg),
// U = qx.wu^T * (sx*su), each summed along K in one running sum; bitwise
// equal to two BF16 launch_gemm calls + launch_silu_mul whenever those GEMMs
// sum along K as well (always when I >= H; see gemm_splits_k).
hipError_t launch_gemm_swiglu(const uint8_t* qx, const uint8_t* wg, const uint8_t* wu,
                              uint8_t* qh, int64_t M, int64_t I, int64_t H,
                              const float* sx, const float* sg, const float* su,
                              const float* sh, int accum, int num_cus, hipStream_t stream);

}  // namespace fp8mot
