/*
 * fp8mot.h -- C ABI of libfp8mot: the static per-tensor FP8 (OCP E4M3FN)
 * W8A8 Linear stack of a Mixture-of-Transformers decoder tower, on AMD
 * MI355X (gfx950).
 *
 * Sources (the passages each call follows are cited at the call):
 *  [MC]  model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN + moving-average
 *        activation observer": header paragraph and section "Scheme".
 *  [PR]  pull request "Load static FP8 Cosmos3 Nano/Super checkpoints without
 *        re-quantizing them" (TensorRT-LLM 17476): sections "Description",
 *        "What changed", "Supported surface, and what is refused", and the
 *        commit messages.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    owned by the caller; the library allocates nothing and keeps no
 *    per-call state (the one exception is the fixed scratch array behind
 *    gated_mlp_fp8_noalloc, see there).  Tensors are dense and contiguous (row-major); a
 *    strided tensor must be rejected by the caller before it gets here
 *    ([PR] first commit message: strided inputs are refused, not copied).
 *  - BF16 tensors are passed as uint16_t bit patterns, FP8 tensors as uint8_t
 *    E4M3FN codes (bias 7, no infinities, 0x7F/0xFF are NaN, max 448).
 *  - Every scale is a `const float*` DEVICE pointer to one FP32 scalar.  The
 *    library never reads a scale on the host: a host read would synchronize
 *    the device on the hot path ([PR] "What changed": the shared-scale
 *    invariant is validated once when the weights are loaded, and no scale
 *    is read during the forward pass).  A NULL scale asks for
 *    dynamic quantization, which the static path refuses
 *    (FP8MOT_ERR_UNSUPPORTED; [PR] "What changed": dynamic quantization is
 *    rejected explicitly).
 *  - Scales must be finite and > 0; that is validated once at load with
 *    fp8_check_shared_scale / by the caller, not per call.
 *  - Calls are asynchronous on `stream`.  The return code covers argument
 *    validation and kernel launch, not kernel completion.  Nothing is
 *    launched when a call returns an error.
 *  - Base pointers of tensors must be 16-byte aligned (128-bit loads and
 *    stores); otherwise FP8MOT_ERR_MISALIGNED -- a refusal, not a slow path
 *    ([PR] "Supported surface, and what is refused": an unsupported case is
 *    refused outright rather than served by a silent fallback).
 *  - Sizes are int64_t element counts.  Negative sizes are
 *    FP8MOT_ERR_INVALID_ARG; an empty tensor (a zero size) is a valid no-op
 *    and then data pointers may be NULL.
 *  - GEMM size limits (fp8_linear and every call built on it): M, N, K at
 *    most INT32_MAX; 256 * K below 0x7FFFF000 (K <= 8,388,576); 256 output
 *    rows below 0x7FFFF000 bytes (row length ldc = N, or the ldc argument,
 *    times 1, 2 or 4 bytes for FP8, BF16, FP32 output); at most INT32_MAX
 *    tiles of 128 x 64.  The kernels address one tile's rows with 32-bit
 *    offsets; larger sizes are FP8MOT_ERR_INVALID_ARG, never wrapped.
 *  - Only gfx950 devices are supported; any other device gives
 *    FP8MOT_ERR_UNSUPPORTED.
 *  - The library is reentrant: calls on different streams may overlap.
 */
#ifndef FP8MOT_H
#define FP8MOT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8MOT_OK = 0,
  FP8MOT_ERR_INVALID_ARG = 1,    /* NULL pointer, negative or too large size, K % 16 != 0, bad enum, non-finite c */
  FP8MOT_ERR_MISALIGNED = 2,     /* a tensor base pointer is not 16-byte aligned */
  FP8MOT_ERR_SCALE_MISMATCH = 3, /* a shared-quantization group's input scales differ */
  FP8MOT_ERR_UNSUPPORTED = 4,    /* NULL scale (dynamic quantization) or non-gfx950 device */
  FP8MOT_ERR_HIP = 5,            /* a HIP runtime call or a kernel launch failed */
  FP8MOT_ERR_WORKSPACE = 6,      /* workspace NULL, misaligned or smaller than required */
  FP8MOT_ERR_TOO_LARGE = 7       /* sizes exceed the allocation-free entry point's scratch */
} fp8mot_status;

/* Bytes of device scratch behind gated_mlp_fp8_noalloc (one copy per device,
 * held by the library until the process ends). */
#define FP8MOT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Output kind of fp8_linear. */
typedef enum {
  FP8MOT_OUT_BF16 = 0, /* y = bf16_rne(acc * (s_x * s_w)), uint16_t [M, N] */
  FP8MOT_OUT_FP8 = 1,  /* y = e4m3(acc * (s_x * s_w) / s_y), uint8_t [M, N] */
  FP8MOT_OUT_F32 = 2   /* y = acc * (s_x * s_w) before any output rounding, float [M, N] */
} fp8mot_out;

/* Accumulation engine of the FP8 GEMMs (fp8_linear and the composites).
 *
 * FP8MOT_ACC_EXACT: the FP8 codes are decoded exactly to F16 in the kernel
 *   and multiplied on the F16 matrix cores; products are accumulated to FP32
 *   precision (|y - alpha*S| stays far inside 1e-5 * alpha * sum|terms|).
 *   Peak is the F16 MFMA rate (2.5 PFLOP/s dense on MI355X).
 * FP8MOT_ACC_FP8_MFMA: the native FP8 matrix-core instruction at twice that
 *   rate.  On gfx950 the FP8 MFMA sums each group of 8 consecutive K products
 *   on a grid 13 bits below the group's largest product (smaller products are
 *   truncated toward zero) before adding the group to the FP32 accumulator;
 *   the per-output error is bounded by alpha * sum over groups of
 *   7 * 2^(e_max(group) - 13) and reaches ~1e-4 of sum|terms| on adversarial
 *   inputs (about 5e-5 on Gaussian activations and weights).
 * The two engines give different (each deterministic) results. */
typedef enum {
  FP8MOT_ACC_EXACT = 0,
  FP8MOT_ACC_FP8_MFMA = 1
} fp8mot_acc;

/* Observer mode of fp8_observe. */
typedef enum {
  FP8MOT_OBS_MAX = 0,       /* running max of the per-call amax */
  FP8MOT_OBS_MOVING_AVG = 1 /* moving average of the per-call amax */
} fp8mot_obs;

/* Observer state, 16 bytes in device memory.  An all-zero state is a fresh
 * observer (the caller zero-fills it once).  `m` is the observed value,
 * `count` the number of calls folded in; `pending` (the call's running amax)
 * and `arrived` (the call's workgroups that have added theirs) are the
 * library's own reduction slots and are back at zero after each call.  Calls
 * on one state must not overlap (use one stream, or one state per stream). */
typedef struct {
  float m;
  int32_t count;
  uint32_t pending;
  uint32_t arrived;
} fp8mot_observer_state;

/* ------------------------------------------------------------------ */
/* Library                                                             */
/* ------------------------------------------------------------------ */

/* Checks that `device` is a gfx950 GPU and caches that result.  Optional:
 * every call checks the current device itself.  Returns FP8MOT_OK,
 * FP8MOT_ERR_UNSUPPORTED (other architecture) or FP8MOT_ERR_HIP. */
int fp8mot_init(int device);

/* Static message for a status code (never NULL). */
const char* fp8mot_status_string(int status);

/* Number of activation-quantization launches made by this process so far
 * (fp8_quant_static, and the one inside each composite).  A test hook for
 * the single-quantization property: a composite call adds exactly 1. */
uint64_t fp8mot_debug_quant_launches(void);

/* Measurement aid, not a step of the path: the read/write ceiling of the
 * HBM-bound kernels' byte mix.  Reads a[0..n) (and b[0..n) when b is not
 * NULL) as 16-bit words and writes out[0..n) = the low byte of a[i] (or of
 * a[i] ^ b[i]): 2 bytes read + 1 written per element like fp8_quant_static,
 * or 4 + 1 like silu_mul_2in_fp8, with their access pattern and grid and no
 * arithmetic.  a, b: [n] 16-byte aligned; out: [n] 16-byte aligned.
 * Refusals as fp8_quant_static (no scale). */
int fp8mot_rw_ceiling(const uint16_t* a, const uint16_t* b, uint8_t* out, int64_t n,
                      hipStream_t stream);

/* Measurement aid, not a step of the path: the rate the matrix cores sustain
 * on given FP8 data with nothing else in the loop (no copies, LDS, decodes or
 * epilogue).  MI355X's clock, and with it the MFMA rate, falls under its
 * power limit by an amount that depends on how much the operand bits toggle,
 * so the GEMM kernels are measured against this rather than the published
 * dense peaks alone.  Every wave takes four A fragments from a[0..na) and
 * four B fragments from b[0..nb) (E4M3 codes, each lane its own, indices
 * wrapped), then issues 8 * iters MFMAs on four accumulators:
 * accum = FP8MOT_ACC_EXACT: v_mfma_f32_32x32x16_f16 on the codes decoded
 * exactly to F16 (2*32*32*16 FLOP each); FP8MOT_ACC_FP8_MFMA: the native
 * v_mfma_scale_f32_32x32x64_f8f6f4 (2*32*32*64 FLOP each).  Grid: one
 * 512-thread workgroup per CU.  sink: one device float, written only if the
 * products sum to a sentinel that finite data never reaches.  *flops (host)
 * receives the launch's FLOP count.  Refusals: a NULL pointer, na or nb < 64,
 * iters < 1 or another accum -> FP8MOT_ERR_INVALID_ARG, before any device
 * access. */
int fp8mot_mfma_ceiling(const uint8_t* a, int64_t na, const uint8_t* b, int64_t nb,
                        int64_t iters, int accum, float* sink, double* flops,
                        hipStream_t stream);

/* Conversion of fp8mot_convert_f32. */
typedef enum {
  FP8MOT_CONV_E4M3_PACKED = 0, /* packed gfx950 conversion after a NaN-propagating clamp to
                                  +-448, NaN bytes set to 0x7F: the quantize and SwiGLU
                                  kernels' bodies and the GEMMs' FP8 output */
  FP8MOT_CONV_E4M3_INT = 1,    /* integer round-to-nearest-even on the bit pattern: the
                                  elementwise kernels' tails */
  FP8MOT_CONV_BF16 = 2         /* packed gfx950 BF16 conversion: the GEMM epilogues */
} fp8mot_conv;

/* Verification aid, not a step of the path: the FP32 -> E4M3 and FP32 ->
 * BF16 conversions of the path's kernels, applied to any FP32 input, so that
 * they can be checked on every FP32 bit pattern against the encoding rules
 * ([MC] "Scheme": E4M3 with round to nearest even; the library saturates to
 * +-448, maps NaN to 0x7F and keeps the sign of zero; BF16 round to nearest
 * even, NaN stays NaN).
 *   kind FP8MOT_CONV_E4M3_PACKED or FP8MOT_CONV_E4M3_INT:
 *     out: uint8_t [n], out[i] = the E4M3 code of x[i];
 *   kind FP8MOT_CONV_BF16:
 *     out: uint16_t [n], out[i] = the BF16 bits of x[i].
 * x: float [n], 16-byte aligned; out 16-byte aligned.  n must be a multiple
 * of 4 (the kernels convert four values at a time); n == 0 is a no-op.
 * Refusals: n < 0, n % 4 != 0, another kind, or (n > 0) a NULL pointer ->
 * FP8MOT_ERR_INVALID_ARG; a misaligned pointer -> FP8MOT_ERR_MISALIGNED. */
int fp8mot_convert_f32(const float* x, void* out, int64_t n, int kind, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Steps of the hot path                                               */
/* ------------------------------------------------------------------ */

/* Static activation quantization ([MC] "Scheme": FP8 E4M3 activations with
 * one static per-tensor scale; [PR] "What changed": the shared activation is
 * quantized once and the FP8 tensor is handed to every projection).
 *   q[i] = e4m3(fp32(x[i]) / *d_scale)
 * with one correctly rounded FP32 division and round-to-nearest-even E4M3
 * encoding that saturates to +-448 (NaN -> 0x7F, the sign of zero kept).
 * x: BF16 [n], q: E4M3 [n] (flat; any rank). */
int fp8_quant_static(const uint16_t* x, uint8_t* q, int64_t n,
                     const float* d_scale, hipStream_t stream);

/* FP8 Linear, one projection with its own weight and weight scale
 * ([PR] "Description": each projection keeps s_i * qW_i, no re-quantization
 * onto max(s); commit messages: each Linear applies its own scale in the
 * GEMM epilogue).
 *   acc[m,n] = sum_k e4m3_value(qx[m,k]) * e4m3_value(qw[n,k])  (FP32 accumulation)
 *   alpha    = fp32(*d_sx * *d_sw)
 *   y[m,n]   = per `out_kind` (see fp8mot_out), acc * alpha first.
 * qx: E4M3 [M, K] row-major; qw: E4M3 [N, K] row-major (out x in, K
 * contiguous); y: [M, N] row-major, contiguous (leading dimension N).
 * K must be a multiple of 16.  d_sy is used only for FP8MOT_OUT_FP8 (NULL
 * there is FP8MOT_ERR_UNSUPPORTED) and ignored otherwise.  K == 0 writes
 * zeros.  `accum` selects the engine (fp8mot_acc).  Order of the FP32 sum:
 * along K, except for a GEMM with K > N whose 128-row output tiles (128x128,
 * or 128x64 when even those are too few) give no CU more than one, where the
 * 128-K blocks at even and at odd
 * positions are summed separately and the two sums added at the end (both
 * orders are FP32 accumulation of the same exact products).  The order
 * depends on (M, N, K) only, so equal shapes give equal bits. */
int fp8_linear(const uint8_t* qx, const uint8_t* qw, void* y, int64_t M,
               int64_t N, int64_t K, const float* d_sx, const float* d_sw,
               int out_kind, const float* d_sy, int accum, hipStream_t stream);

/* Two-input SwiGLU with direct FP8 emission ([PR] "What changed" and the
 * first commit message: SiLU(G) * U from two separate tensors, quantized for
 * the FP8 down projection; flat indexing, rank-agnostic).
 *   q[i] = e4m3(silu(g[i]) * u[i] / *d_s_out),  silu(g) = g / (1 + exp(-g))
 * evaluated in FP32.  g, u: BF16 [n]; q: E4M3 [n]. */
int silu_mul_2in_fp8(const uint16_t* g, const uint16_t* u, uint8_t* q,
                     int64_t n, const float* d_s_out, hipStream_t stream);

/* The same with the swiglu_alpha / swiglu_beta variant ([PR] commit message
 * on swiglu_alpha / swiglu_beta: alpha is a gain inside the sigmoid, beta an
 * offset on up):
 *   q[i] = e4m3(g[i] * sigmoid(alpha * g[i]) * (u[i] + beta) / *d_s_out)
 * in FP32.  A zero beta leaves u untouched, so (alpha, beta) = (1, 0) gives
 * exactly the codes of silu_mul_2in_fp8.  Non-finite alpha or beta is
 * FP8MOT_ERR_INVALID_ARG; other arguments as silu_mul_2in_fp8. */
int silu_mul_2in_fp8_ab(const uint16_t* g, const uint16_t* u, uint8_t* q,
                        int64_t n, const float* d_s_out, float alpha, float beta,
                        hipStream_t stream);

/* One-input SwiGLU with gate and up adjacent in one tensor ([PR] commit
 * message: silu_and_mul needs gate and up adjacent; the two-input form exists
 * because separate projections have no such tensor).  x: BF16 [rows, 2*inter]
 * whose row r holds the inter gate values, then the inter up values;
 * q: E4M3 [rows, inter]:
 *   q[r, c] = e4m3(g * sigmoid(alpha g) * (u + beta) / *d_s_out),
 *   g = x[r, c], u = x[r, inter + c],
 * bit for bit what silu_mul_2in_fp8_ab gives on the two halves.  x and q
 * 16-byte aligned (FP8MOT_ERR_MISALIGNED); rows, inter >= 0; any inter (a
 * multiple of 16 takes the vector path). */
int silu_mul_fp8(const uint16_t* x, uint8_t* q, int64_t rows, int64_t inter,
                 const float* d_s_out, float alpha, float beta, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Per-row FP8 (per-channel weights, per-token activations)            */
/* ------------------------------------------------------------------ */

/* Per-row dynamic quantization ([MC] section 3.2: the per-channel weight /
 * per-token activation builds; the runtime FP8 path quantizes weights per
 * output channel at load and activations per token at run time).  For each
 * row r of x (BF16 [rows, K]):
 *   d_scales[r] = fp32(max_k |x[r,k]|) / 448      (FP32 division)
 *   q[r,k]      = e4m3(fp32(x[r,k]) / d_scales[r]) (IEEE FP32 division)
 * A zero row gets scale 0 and keeps its signed zeros; a row holding a NaN
 * gets a NaN scale and NaN codes.  Used for per-token activations (rows =
 * tokens) and, at load time, per-channel weights (rows = output channels).
 * K must be a multiple of 16 (FP8MOT_ERR_INVALID_ARG); x, q 16-byte aligned
 * (FP8MOT_ERR_MISALIGNED); d_scales: FP32 [rows], caller-owned device memory.
 * rows == 0 does nothing; K == 0 writes scale 0 for every row (an empty row
 * is a zero row) and then x and q may be NULL. */
int fp8_quant_per_row(const uint16_t* x, uint8_t* q, float* d_scales,
                      int64_t rows, int64_t K, hipStream_t stream);

/* FP8 GEMM with per-row scales on both operands:
 *   y[m,n] = fp32( acc[m,n] * fp32(d_sx[m] * d_sw[n]) ),
 *   acc[m,n] = sum_k dec(qx[m,k]) * dec(qw[n,k])   (engine per `accum`)
 * d_sx: FP32 [M] (per token), d_sw: FP32 [N] (per output channel), both
 * device memory, 16-byte aligned.  out_kind: FP8MOT_OUT_BF16 or
 * FP8MOT_OUT_F32 (FP8 output is FP8MOT_ERR_UNSUPPORTED).  Other arguments and
 * refusals as fp8_linear. */
int fp8_linear_rowwise(const uint8_t* qx, const uint8_t* qw, void* y, int64_t M,
                       int64_t N, int64_t K, const float* d_sx, const float* d_sw,
                       int out_kind, int accum, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Fused-topology comparison (what the split path avoids)              */
/* ------------------------------------------------------------------ */

/* fp8_linear writing into a row-strided output: row m of y starts ldc
 * elements after row m - 1 (ldc >= N), so two projections can write the
 * column slices [:, 0:N) and [:, N:2N) of one [M, 2N] buffer ([PR] "What
 * changed": writing both GEMMs into column slices of one buffer went wrong
 * in the original stack because the GEMM assumed the leading dimension was
 * N).  Elements of y outside [0, M) x [0, N) are not written.  ldc < N is
 * FP8MOT_ERR_INVALID_ARG; other arguments as fp8_linear. */
int fp8_linear_ldc(const uint8_t* qx, const uint8_t* qw, void* y, int64_t M,
                   int64_t N, int64_t K, int64_t ldc, const float* d_sx,
                   const float* d_sw, int out_kind, const float* d_sy, int accum,
                   hipStream_t stream);

/* The failure mode of a fused group that keeps one scale ([PR]
 * "Description": each member re-quantized as FP8-round((s_i * qW_i) /
 * max(s))), for the fused-topology comparison only:
 *   out[k] = e4m3(fp32(fp32(*d_s_member * dec(qw[k])) / max(d_s_group[0..g-1])))
 * qw, out: E4M3 [n], 16-byte aligned; d_s_member: FP32 scalar, d_s_group:
 * FP32 [group_size] (1..64), device memory.  NULL scales are
 * FP8MOT_ERR_UNSUPPORTED. */
int fp8_requantize_onto_max(const uint8_t* qw, uint8_t* out, int64_t n,
                            const float* d_s_member, const float* d_s_group,
                            int group_size, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Composites (one shared quantization, contiguous outputs, no sync)   */
/* ------------------------------------------------------------------ */

/* Bytes of workspace gated_mlp_fp8 needs: qX [M,H] + qH [M,I], each region
 * 256-byte aligned.  Returns 0 for negative sizes. */
size_t gated_mlp_fp8_workspace(int64_t M, int64_t H, int64_t I);

/* Gated MLP with split gate/up ([PR] "What changed": GatedMLP with
 * split_gate_up quantizes the shared activation once and hands both
 * projections the FP8 tensor; SiLU(G)*U emits FP8 at the down input scale).
 *   qX = quant(x; sx); G = linear(qX, wg; sx, sg); U = linear(qX, wu; sx, su)
 *   qH = silu_mul_2in(G, U; sh); y = linear(qH, wd; sh, sd)  (BF16 out)
 * Bitwise equal to those five calls when I >= H (the gate and up GEMMs and
 * the SwiGLU run as one kernel whose epilogue rounds G and U to BF16 and
 * applies the SwiGLU exactly as the separate calls do; G and U are never
 * written).  With H > I and few tiles the separate gate/up fp8_linear calls
 * sum K in two halves (see fp8_linear) while this kernel sums along K, so
 * an SwiGLU code can then differ by one step.
 * x: [M, H]; wg, wu: [I, H]; wd: [H, I];
 * y: [M, H].  H and I multiples of 16.  ws: device workspace of at least
 * gated_mlp_fp8_workspace(M, H, I) bytes, 256-byte aligned.  `accum`
 * selects the GEMM engine (fp8mot_acc) of all three GEMMs.  I == 0 (empty
 * weights, whose pointers may be NULL) writes y = 0, the down projection of
 * an empty sum; M == 0 or H == 0 writes nothing. */
int gated_mlp_fp8(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                  const float* d_sx, const uint8_t* wg, const float* d_sg,
                  const uint8_t* wu, const float* d_su, const float* d_sh,
                  const uint8_t* wd, const float* d_sd, uint16_t* y, void* ws,
                  size_t ws_bytes, int accum, hipStream_t stream);

/* gated_mlp_fp8 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launches and bitwise the same y, with qX and qH kept in a scratch
 * array the library holds per device (FP8MOT_NOALLOC_SCRATCH_BYTES, a
 * file-scope device array whose address is looked up once per device)
 * instead of a caller workspace.  The call allocates nothing.
 * Limit: gated_mlp_fp8_workspace(M, H, I) <= FP8MOT_NOALLOC_SCRATCH_BYTES
 * (64 MiB: M * (H + I) up to about 64M codes, e.g. M = 4096, H = 4096,
 * I = 12288), else FP8MOT_ERR_TOO_LARGE and nothing is launched.
 * Every call on one device shares that device's scratch: calls that overlap
 * on one GPU (different streams, or different threads without ordering) race
 * on it and must be serialized by the caller.  Nothing in the scratch needs
 * to start at zero (each call overwrites the qX and qH it reads).  Other
 * arguments, refusals and the engine choice as gated_mlp_fp8. */
int gated_mlp_fp8_noalloc(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                          const float* d_sx, const uint8_t* wg, const float* d_sg,
                          const uint8_t* wu, const float* d_su, const float* d_sh,
                          const uint8_t* wd, const float* d_sd, uint16_t* y, int accum,
                          hipStream_t stream);

/* The gate/up half of the gated MLP from an already quantized activation
 * ([PR] "What changed": one quantized activation handed to both
 * projections; the two-input SwiGLU emits FP8 for the down projection):
 *   qh = silu_mul_2in_fp8(linear(qx, wg; sx, sg), linear(qx, wu; sx, su); sh)
 * (bitwise when I >= H, as for gated_mlp_fp8), computed by one kernel that
 * shares each qx tile between the two GEMMs and never writes G or U.  qx: E4M3 [M, H]; wg, wu: E4M3 [I, H];
 * qh: E4M3 [M, I].  H and I multiples of 16.  `accum` per fp8mot_acc. */
int fp8_gate_up_swiglu(const uint8_t* qx, const uint8_t* wg, const float* d_sx,
                       const float* d_sg, const uint8_t* wu, const float* d_su,
                       const float* d_sh, uint8_t* qh, int64_t M, int64_t I,
                       int64_t H, int accum, hipStream_t stream);

/* Bytes of workspace qkv_fp8 needs: qX [M, H], 256-byte aligned. */
size_t qkv_fp8_workspace(int64_t M, int64_t H);

/* Split Q/K/V with one shared activation quantization ([PR] "What changed":
 * Attention with share_qkv_input_quant; "It is also faster": split
 * projections give contiguous outputs).
 *   qX = quant(x; sx); yq = linear(qX, wq; sx, sq); yk = ...; yv = ...
 * x: [M, H]; wq: [Nq, H]; wk: [Nk, H]; wv: [Nv, H]; yq: [M, Nq], yk: [M, Nk],
 * yv: [M, Nv], three separate contiguous BF16 tensors.  H multiple of 16.
 * The three GEMMs run as one grouped launch, or as three launches when
 * fp8_linear would split K for one of them; either way bitwise what three
 * fp8_linear calls give.  A member with N == 0 is skipped and its pointers may be NULL.
 * H == 0 quantizes nothing (x, the weights and ws may be NULL) and writes each
 * projection's epilogue of an empty sum, zero; M == 0 writes nothing.
 * Cross-attention, where k/v read a different tensor than q, must not use
 * this call: quantize each input separately and use fp8_linear.  `accum`
 * selects the GEMM engine (fp8mot_acc). */
int qkv_fp8(const uint16_t* x, int64_t M, int64_t H, const float* d_sx,
            const uint8_t* wq, int64_t Nq, const float* d_sq,
            const uint8_t* wk, int64_t Nk, const float* d_sk,
            const uint8_t* wv, int64_t Nv, const float* d_sv, uint16_t* yq,
            uint16_t* yk, uint16_t* yv, void* ws, size_t ws_bytes, int accum,
            hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Calibration                                                         */
/* ------------------------------------------------------------------ */

/* Folds one calibration call into an observer ([MC] header and "Scheme":
 * static input scales from the global max of the activations, or from a
 * moving average of the per-call maxima with constant 0.01).
 *   a = max |x[i]|   (NaN if any x[i] is NaN)
 *   first call: m = a
 *   FP8MOT_OBS_MAX:        m = max(m, a)            (NaN propagates)
 *   FP8MOT_OBS_MOVING_AVG: m = m + c * (a - m)      (three FP32 roundings, no FMA)
 * x: BF16 [n], n >= 1 (an empty call has no maximum to fold, so n == 0 is
 * FP8MOT_ERR_INVALID_ARG, the one exception to the empty-tensor rule above).
 * d_state: device fp8mot_observer_state (zero-filled
 * before the first call; 16-byte aligned).  `c` is used by the moving
 * average only and must be finite.  Calls on one state must be
 * stream-ordered. */
int fp8_observe(const uint16_t* x, int64_t n, void* d_state, int mode,
                float c, hipStream_t stream);

/* Same as fp8_observe with a = max |silu(g[i]) * u[i]| (FP32 evaluation as in
 * silu_mul_2in_fp8): calibrates the down projection's input scale from the
 * gate/up outputs without materializing the product. */
int fp8_observe_swiglu(const uint16_t* g, const uint16_t* u, int64_t n,
                       void* d_state, int mode, float c, hipStream_t stream);

/* *d_scale = fp32(state.m / 448): the static per-tensor scale. */
int fp8_scale_from_state(const void* d_state, float* d_scale,
                         hipStream_t stream);

/* Load-time check of a shared-quantization group ([PR] "What changed": the
 * projections sharing one quantized activation must carry the same
 * calibrated input_scale; validated when the weights are loaded, not in the
 * forward pass).
 * h_scales: HOST array of n >= 1 scales.  FP8MOT_OK iff all are finite,
 * > 0 and bitwise equal; FP8MOT_ERR_SCALE_MISMATCH if they differ;
 * FP8MOT_ERR_INVALID_ARG for NULL, n < 1, or a non-finite or non-positive
 * scale.  Pure host code: usable without a GPU. */
int fp8_check_shared_scale(const float* h_scales, int n);

#ifdef __cplusplus
}
#endif

#endif /* FP8MOT_H */
