// C ABI of libfp8mot (declared in include/fp8mot.h): argument validation,
// device checks, workspace layout and the composites.  Every step of the
// path runs in this library's kernels; validation happens before any HIP
// call, so a refused call launches nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/fp8mot.h"
#include "kernels.h"

using namespace fp8mot;

namespace {

std::atomic<uint64_t> g_quant_launches{0};

constexpr int kMaxDevices = 64;
// per device: 0 = not checked, 1 = gfx950, 2 = unsupported
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

int check_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return FP8MOT_ERR_UNSUPPORTED;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8MOT_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    st = ok ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FP8MOT_OK : FP8MOT_ERR_UNSUPPORTED;
}

// Checks the current device; on success stores its CU count.
int current_device(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8MOT_ERR_HIP;
  const int st = check_device(dev);
  if (st == FP8MOT_OK) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return st;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8MOT_OK : FP8MOT_ERR_HIP; }

// Workgroup budget of the grid-stride elementwise kernels: 8 per CU.  The
// launchers scale it per kernel (quantize and SwiGLU use twice as many, the
// amax reductions a quarter), as measured on MI355X.
int ew_blocks(int cus) { return cus * 8; }

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

struct MlpLayout {
  size_t qx, qh, total;
};

// qX [M, H] then qH [M, I]; G and U never leave the fused gate/up kernel
MlpLayout mlp_layout(int64_t M, int64_t H, int64_t I) {
  MlpLayout l;
  l.qx = 0;
  l.qh = l.qx + round256((size_t)M * H);
  l.total = l.qh + round256((size_t)M * I);
  return l;
}

// Validation shared by the GEMM entry points.
// The GEMM kernels address one tile's operand rows (at most 256 rows of K
// codes) and its output rows (at most 256 rows of ldc elements of esz bytes)
// with 32-bit byte offsets that must stay below their out-of-range sentinel
// (0x7FFFFFF0), and number their tiles (128 x 64 at the smallest) with a
// 32-bit workgroup index.  Larger sizes are refused rather than wrapped.
constexpr int64_t kTileWindowBytes = 0x7FFFF000;
bool gemm_sizes_ok(int64_t M, int64_t N, int64_t K, int64_t ldc, int esz) {
  if (256 * K >= kTileWindowBytes) return false;
  if (256 * ldc * esz >= kTileWindowBytes) return false;
  return ((M + 127) / 128) * ((N + 63) / 64) <= INT32_MAX;
}

int out_bytes(int out_kind) {
  return out_kind == FP8MOT_OUT_FP8 ? 1 : (out_kind == FP8MOT_OUT_BF16 ? 2 : 4);
}

int check_linear(const uint8_t* qx, const uint8_t* qw, const void* y, int64_t M,
                 int64_t N, int64_t K, const float* sx, const float* sw,
                 int out_kind, const float* sy, int accum) {
  if (out_kind < 0 || out_kind > 2) return FP8MOT_ERR_INVALID_ARG;
  if (accum != FP8MOT_ACC_EXACT && accum != FP8MOT_ACC_FP8_MFMA) return FP8MOT_ERR_INVALID_ARG;
  if (sx == nullptr || sw == nullptr) return FP8MOT_ERR_UNSUPPORTED;
  if (out_kind == FP8MOT_OUT_FP8 && sy == nullptr) return FP8MOT_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || (K % 16) != 0) return FP8MOT_ERR_INVALID_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return FP8MOT_ERR_INVALID_ARG;
  if (!gemm_sizes_ok(M, N, K, N, out_bytes(out_kind))) return FP8MOT_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8MOT_OK;
  if (y == nullptr || (K > 0 && (qx == nullptr || qw == nullptr)))
    return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(qx) || !aligned16(qw)) return FP8MOT_ERR_MISALIGNED;
  return FP8MOT_OK;
}

}  // namespace

extern "C" {

int fp8mot_init(int device) {
  if (device < 0 || device >= kMaxDevices) return FP8MOT_ERR_INVALID_ARG;
  return check_device(device);
}

const char* fp8mot_status_string(int status) {
  switch (status) {
    case FP8MOT_OK: return "ok";
    case FP8MOT_ERR_INVALID_ARG: return "invalid argument (NULL pointer, negative or too large size, K % 16 != 0, bad enum or non-finite constant)";
    case FP8MOT_ERR_MISALIGNED: return "tensor base pointer not 16-byte aligned";
    case FP8MOT_ERR_SCALE_MISMATCH: return "input scales of a shared-quantization group differ";
    case FP8MOT_ERR_UNSUPPORTED: return "unsupported: NULL scale (dynamic quantization) or non-gfx950 device";
    case FP8MOT_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case FP8MOT_ERR_WORKSPACE: return "workspace NULL, misaligned or too small";
    case FP8MOT_ERR_TOO_LARGE: return "sizes need more scratch than the allocation-free entry point holds (FP8MOT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

uint64_t fp8mot_debug_quant_launches(void) { return g_quant_launches.load(); }

int fp8mot_rw_ceiling(const uint16_t* a, const uint16_t* b, uint8_t* out, int64_t n,
                      hipStream_t stream) {
  if (n < 0) return FP8MOT_ERR_INVALID_ARG;
  if (n == 0) return FP8MOT_OK;
  if (a == nullptr || out == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(out) || (b != nullptr && !aligned16(b)))
    return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_rw_ceiling(a, b, out, n, ew_blocks(cus), stream));
}

int fp8mot_mfma_ceiling(const uint8_t* a, int64_t na, const uint8_t* b, int64_t nb,
                        int64_t iters, int accum, float* sink, double* flops,
                        hipStream_t stream) {
  if (a == nullptr || b == nullptr || sink == nullptr || flops == nullptr || na < 64 ||
      nb < 64 || iters < 1)
    return FP8MOT_ERR_INVALID_ARG;
  if (accum != FP8MOT_ACC_EXACT && accum != FP8MOT_ACC_FP8_MFMA) return FP8MOT_ERR_INVALID_ARG;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  *flops = mfma_ceiling_flops(cus, iters, accum);
  return hip_status(launch_mfma_ceiling(a, na, b, nb, iters, accum, sink, cus, stream));
}

int fp8mot_convert_f32(const float* x, void* out, int64_t n, int kind, hipStream_t stream) {
  if (n < 0 || n % 4 != 0) return FP8MOT_ERR_INVALID_ARG;
  if (kind != FP8MOT_CONV_E4M3_PACKED && kind != FP8MOT_CONV_E4M3_INT && kind != FP8MOT_CONV_BF16)
    return FP8MOT_ERR_INVALID_ARG;
  if (n == 0) return FP8MOT_OK;
  if (x == nullptr || out == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_convert_f32(x, out, n, kind, ew_blocks(cus), stream));
}

int fp8_quant_static(const uint16_t* x, uint8_t* q, int64_t n,
                     const float* d_scale, hipStream_t stream) {
  if (d_scale == nullptr) return FP8MOT_ERR_UNSUPPORTED;
  if (n < 0) return FP8MOT_ERR_INVALID_ARG;
  if (n == 0) return FP8MOT_OK;
  if (x == nullptr || q == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  g_quant_launches.fetch_add(1);
  return hip_status(launch_quant_static(x, q, n, d_scale, ew_blocks(cus), stream));
}

int fp8_linear(const uint8_t* qx, const uint8_t* qw, void* y, int64_t M,
               int64_t N, int64_t K, const float* d_sx, const float* d_sw,
               int out_kind, const float* d_sy, int accum, hipStream_t stream) {
  int st = check_linear(qx, qw, y, M, N, K, d_sx, d_sw, out_kind, d_sy, accum);
  if (st != FP8MOT_OK || M == 0 || N == 0) return st;
  int cus = 0;
  st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_gemm(qx, qw, y, M, N, K, d_sx, d_sw, out_kind, d_sy, accum, cus, stream));
}

int fp8_linear_rowwise(const uint8_t* qx, const uint8_t* qw, void* y, int64_t M,
                       int64_t N, int64_t K, const float* d_sx, const float* d_sw,
                       int out_kind, int accum, hipStream_t stream) {
  if (out_kind == FP8MOT_OUT_FP8) return FP8MOT_ERR_UNSUPPORTED;
  int st = check_linear(qx, qw, y, M, N, K, d_sx, d_sw, out_kind, nullptr, accum);
  if (st != FP8MOT_OK || M == 0 || N == 0) return st;
  if (!aligned16(d_sx) || !aligned16(d_sw)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  // out kinds 3 / 4 of the launcher: BF16 / FP32 with per-row scales
  const int kind = out_kind == FP8MOT_OUT_BF16 ? 3 : 4;
  return hip_status(launch_gemm(qx, qw, y, M, N, K, d_sx, d_sw, kind, nullptr, accum, cus, stream));
}

int fp8_linear_ldc(const uint8_t* qx, const uint8_t* qw, void* y, int64_t M,
                   int64_t N, int64_t K, int64_t ldc, const float* d_sx,
                   const float* d_sw, int out_kind, const float* d_sy, int accum,
                   hipStream_t stream) {
  int st = check_linear(qx, qw, y, M, N, K, d_sx, d_sw, out_kind, d_sy, accum);
  if (st != FP8MOT_OK) return st;
  if (ldc < N || ldc > INT32_MAX) return FP8MOT_ERR_INVALID_ARG;
  if (M > 0 && ldc > INT64_MAX / M) return FP8MOT_ERR_INVALID_ARG;
  if (!gemm_sizes_ok(M, N, K, ldc, out_bytes(out_kind))) return FP8MOT_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8MOT_OK;
  int cus = 0;
  st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_gemm(qx, qw, y, M, N, K, d_sx, d_sw, out_kind, d_sy, accum, cus,
                                stream, ldc));
}

int fp8_requantize_onto_max(const uint8_t* qw, uint8_t* out, int64_t n,
                            const float* d_s_member, const float* d_s_group,
                            int group_size, hipStream_t stream) {
  if (d_s_member == nullptr || d_s_group == nullptr) return FP8MOT_ERR_UNSUPPORTED;
  if (n < 0 || group_size < 1 || group_size > 64) return FP8MOT_ERR_INVALID_ARG;
  if (n == 0) return FP8MOT_OK;
  if (qw == nullptr || out == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(qw) || !aligned16(out)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_requant_onto_max(qw, out, n, d_s_member, d_s_group, group_size,
                                            ew_blocks(cus), stream));
}

int fp8_quant_per_row(const uint16_t* x, uint8_t* q, float* d_scales,
                      int64_t rows, int64_t K, hipStream_t stream) {
  if (rows < 0 || K < 0 || (K % 16) != 0) return FP8MOT_ERR_INVALID_ARG;
  if (rows > 0 && K > INT64_MAX / rows) return FP8MOT_ERR_INVALID_ARG;
  if (rows == 0) return FP8MOT_OK;
  // K == 0: empty rows, each a zero row (scale 0); x and q may be NULL
  if (d_scales == nullptr || (K > 0 && (x == nullptr || q == nullptr)))
    return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_quant_per_row(x, q, d_scales, rows, K, ew_blocks(cus), stream));
}

int silu_mul_2in_fp8_ab(const uint16_t* g, const uint16_t* u, uint8_t* q,
                        int64_t n, const float* d_s_out, float alpha, float beta,
                        hipStream_t stream) {
  if (d_s_out == nullptr) return FP8MOT_ERR_UNSUPPORTED;
  if (n < 0 || !std::isfinite(alpha) || !std::isfinite(beta)) return FP8MOT_ERR_INVALID_ARG;
  if (n == 0) return FP8MOT_OK;
  if (g == nullptr || u == nullptr || q == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(g) || !aligned16(u) || !aligned16(q)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_silu_mul(g, u, q, n, d_s_out, alpha, beta, ew_blocks(cus), stream));
}

int silu_mul_2in_fp8(const uint16_t* g, const uint16_t* u, uint8_t* q,
                     int64_t n, const float* d_s_out, hipStream_t stream) {
  return silu_mul_2in_fp8_ab(g, u, q, n, d_s_out, 1.0f, 0.0f, stream);
}

int silu_mul_fp8(const uint16_t* x, uint8_t* q, int64_t rows, int64_t inter,
                 const float* d_s_out, float alpha, float beta, hipStream_t stream) {
  if (d_s_out == nullptr) return FP8MOT_ERR_UNSUPPORTED;
  if (rows < 0 || inter < 0 || !std::isfinite(alpha) || !std::isfinite(beta))
    return FP8MOT_ERR_INVALID_ARG;
  if (rows > 0 && inter > INT64_MAX / 2 / rows) return FP8MOT_ERR_INVALID_ARG;
  if (rows == 0 || inter == 0) return FP8MOT_OK;
  if (x == nullptr || q == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_silu_mul_adjacent(x, q, rows, inter, d_s_out, alpha, beta,
                                             ew_blocks(cus), stream));
}

size_t gated_mlp_fp8_workspace(int64_t M, int64_t H, int64_t I) {
  if (M < 0 || H < 0 || I < 0) return 0;
  return mlp_layout(M, H, I).total;
}

}  // extern "C"

namespace {

// Argument checks of the gated MLP (everything but the workspace).
int check_gated_mlp(const uint16_t* x, int64_t M, int64_t H, int64_t I, const float* d_sx,
                    const uint8_t* wg, const float* d_sg, const uint8_t* wu,
                    const float* d_su, const float* d_sh, const uint8_t* wd,
                    const float* d_sd, const uint16_t* y, int accum) {
  if (!d_sx || !d_sg || !d_su || !d_sh || !d_sd) return FP8MOT_ERR_UNSUPPORTED;
  if (accum != FP8MOT_ACC_EXACT && accum != FP8MOT_ACC_FP8_MFMA) return FP8MOT_ERR_INVALID_ARG;
  if (M < 0 || H < 0 || I < 0 || (H % 16) != 0 || (I % 16) != 0)
    return FP8MOT_ERR_INVALID_ARG;
  if (M > INT32_MAX || H > INT32_MAX || I > INT32_MAX) return FP8MOT_ERR_INVALID_ARG;
  // gate/up: K = H, FP8 output rows of I; down: K = I, BF16 output rows of H
  if (!gemm_sizes_ok(M, I, H, I, 1) || !gemm_sizes_ok(M, H, I, H, 2)) return FP8MOT_ERR_INVALID_ARG;
  if (M == 0 || H == 0) return FP8MOT_OK;
  // I == 0: the three weights are empty (their pointers may be NULL) and y is
  // the down projection of an empty sum, zero
  if (!x || !y || (I > 0 && (!wg || !wu || !wd))) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || !aligned16(wd) || !aligned16(y))
    return FP8MOT_ERR_MISALIGNED;
  return FP8MOT_OK;
}

// The gated MLP's launches, with qX and qH in `base` laid out by mlp_layout.
int run_gated_mlp(const uint16_t* x, int64_t M, int64_t H, int64_t I, const float* d_sx,
                  const uint8_t* wg, const float* d_sg, const uint8_t* wu, const float* d_su,
                  const float* d_sh, const uint8_t* wd, const float* d_sd, uint16_t* y,
                  uint8_t* base, int accum, int cus, hipStream_t stream) {
  const MlpLayout l = mlp_layout(M, H, I);
  uint8_t* qx = base + l.qx;
  uint8_t* qh = base + l.qh;
  g_quant_launches.fetch_add(1);
  hipError_t e = launch_quant_static(x, qx, M * H, d_sx, ew_blocks(cus), stream);
  // gate and up GEMMs with the SwiGLU-FP8 epilogue in one launch: the same
  // arithmetic, in the same order, as the two BF16 GEMMs and
  // silu_mul_2in_fp8 whenever those GEMMs sum K in one running sum, without
  // writing G and U
  if (e == hipSuccess && I > 0)
    e = launch_gemm_swiglu(qx, wg, wu, qh, M, I, H, d_sx, d_sg, d_su, d_sh, accum, cus, stream);
  if (e == hipSuccess)
    e = launch_gemm(qh, wd, y, M, H, I, d_sh, d_sd, FP8MOT_OUT_BF16, nullptr, accum, cus, stream);
  return hip_status(e);
}

// Scratch of gated_mlp_fp8_noalloc: qX and qH at the offsets of
// gated_mlp_fp8's workspace.  Each device the library runs on holds its own
// copy until the process ends.  Host code never passes `scratch` itself (on
// the host it names a stand-in, not device memory): it passes the device
// address that hipGetSymbolAddress returns for the current device, taken once
// per device and kept in g_scratch_dev.
static __device__ __align__(256) uint8_t scratch[FP8MOT_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

// Device address of the current device's scratch (the caller has checked the
// device: 0 <= dev < kMaxDevices and gfx950).
int scratch_of_device(int dev, uint8_t** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FP8MOT_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch_dev[dev]);
  return FP8MOT_OK;
}

}  // namespace

extern "C" {

int gated_mlp_fp8(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                  const float* d_sx, const uint8_t* wg, const float* d_sg,
                  const uint8_t* wu, const float* d_su, const float* d_sh,
                  const uint8_t* wd, const float* d_sd, uint16_t* y, void* ws,
                  size_t ws_bytes, int accum, hipStream_t stream) {
  int st = check_gated_mlp(x, M, H, I, d_sx, wg, d_sg, wu, d_su, d_sh, wd, d_sd, y, accum);
  if (st != FP8MOT_OK || M == 0 || H == 0) return st;
  if (ws == nullptr || !aligned256(ws) || ws_bytes < mlp_layout(M, H, I).total)
    return FP8MOT_ERR_WORKSPACE;
  int cus = 0;
  st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return run_gated_mlp(x, M, H, I, d_sx, wg, d_sg, wu, d_su, d_sh, wd, d_sd, y,
                       static_cast<uint8_t*>(ws), accum, cus, stream);
}

int gated_mlp_fp8_noalloc(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                          const float* d_sx, const uint8_t* wg, const float* d_sg,
                          const uint8_t* wu, const float* d_su, const float* d_sh,
                          const uint8_t* wd, const float* d_sd, uint16_t* y, int accum,
                          hipStream_t stream) {
  int st = check_gated_mlp(x, M, H, I, d_sx, wg, d_sg, wu, d_su, d_sh, wd, d_sd, y, accum);
  if (st != FP8MOT_OK || M == 0 || H == 0) return st;
  if (mlp_layout(M, H, I).total > FP8MOT_NOALLOC_SCRATCH_BYTES) return FP8MOT_ERR_TOO_LARGE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8MOT_ERR_HIP;
  int cus = 0;
  st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  uint8_t* base = nullptr;
  st = scratch_of_device(dev, &base);
  if (st != FP8MOT_OK) return st;
  return run_gated_mlp(x, M, H, I, d_sx, wg, d_sg, wu, d_su, d_sh, wd, d_sd, y, base, accum,
                       cus, stream);
}

int fp8_gate_up_swiglu(const uint8_t* qx, const uint8_t* wg, const float* d_sx,
                       const float* d_sg, const uint8_t* wu, const float* d_su,
                       const float* d_sh, uint8_t* qh, int64_t M, int64_t I,
                       int64_t H, int accum, hipStream_t stream) {
  if (!d_sx || !d_sg || !d_su || !d_sh) return FP8MOT_ERR_UNSUPPORTED;
  if (accum != FP8MOT_ACC_EXACT && accum != FP8MOT_ACC_FP8_MFMA) return FP8MOT_ERR_INVALID_ARG;
  if (M < 0 || H < 0 || I < 0 || (H % 16) != 0 || (I % 16) != 0)
    return FP8MOT_ERR_INVALID_ARG;
  if (M > INT32_MAX || H > INT32_MAX || I > INT32_MAX) return FP8MOT_ERR_INVALID_ARG;
  if (!gemm_sizes_ok(M, I, H, I, 1)) return FP8MOT_ERR_INVALID_ARG;
  if (M == 0 || I == 0) return FP8MOT_OK;
  if (!qh || (H > 0 && (!qx || !wg || !wu))) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(qx) || !aligned16(wg) || !aligned16(wu) || !aligned16(qh))
    return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_gemm_swiglu(qx, wg, wu, qh, M, I, H, d_sx, d_sg, d_su, d_sh, accum, cus, stream));
}

size_t qkv_fp8_workspace(int64_t M, int64_t H) {
  if (M < 0 || H < 0) return 0;
  return round256((size_t)M * H);
}

int qkv_fp8(const uint16_t* x, int64_t M, int64_t H, const float* d_sx,
            const uint8_t* wq, int64_t Nq, const float* d_sq,
            const uint8_t* wk, int64_t Nk, const float* d_sk,
            const uint8_t* wv, int64_t Nv, const float* d_sv, uint16_t* yq,
            uint16_t* yk, uint16_t* yv, void* ws, size_t ws_bytes, int accum,
            hipStream_t stream) {
  if (!d_sx || !d_sq || !d_sk || !d_sv) return FP8MOT_ERR_UNSUPPORTED;
  if (accum != FP8MOT_ACC_EXACT && accum != FP8MOT_ACC_FP8_MFMA) return FP8MOT_ERR_INVALID_ARG;
  if (M < 0 || H < 0 || Nq < 0 || Nk < 0 || Nv < 0 || (H % 16) != 0)
    return FP8MOT_ERR_INVALID_ARG;
  if (M > INT32_MAX || H > INT32_MAX || Nq > INT32_MAX || Nk > INT32_MAX || Nv > INT32_MAX)
    return FP8MOT_ERR_INVALID_ARG;
  // the grouped launch numbers the tiles of all three members together
  if (!gemm_sizes_ok(M, Nq + Nk + Nv, H, Nq > Nk ? (Nq > Nv ? Nq : Nv) : (Nk > Nv ? Nk : Nv), 2))
    return FP8MOT_ERR_INVALID_ARG;
  if (M == 0) return FP8MOT_OK;
  // a member with N == 0 has nothing to read or write (its pointers may be
  // NULL); with H == 0 neither has x nor a member's weight
  if ((H > 0 && !x) || (Nq > 0 && ((H > 0 && !wq) || !yq)) ||
      (Nk > 0 && ((H > 0 && !wk) || !yk)) || (Nv > 0 && ((H > 0 && !wv) || !yv)))
    return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || (Nq > 0 && (!aligned16(wq) || !aligned16(yq))) ||
      (Nk > 0 && (!aligned16(wk) || !aligned16(yk))) || (Nv > 0 && (!aligned16(wv) || !aligned16(yv))))
    return FP8MOT_ERR_MISALIGNED;
  // H == 0 needs no workspace (qX is empty)
  const size_t need = qkv_fp8_workspace(M, H);
  if (need > 0 && (ws == nullptr || !aligned256(ws) || ws_bytes < need))
    return FP8MOT_ERR_WORKSPACE;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  uint8_t* qx = static_cast<uint8_t*>(ws);
  hipError_t e = hipSuccess;
  if (H > 0) {
    g_quant_launches.fetch_add(1);
    e = launch_quant_static(x, qx, M * H, d_sx, ew_blocks(cus), stream);
  }
  // the three projections in one grouped launch (the non-empty ones): tiles
  // of all three share qX rows in L2 and fill the machine together
  const uint8_t* wb[3];
  void* yb[3];
  const float* sb[3];
  int64_t nb[3];
  int groups = 0;
  const uint8_t* w3[3] = {wq, wk, wv};
  uint16_t* y3[3] = {yq, yk, yv};
  const float* s3[3] = {d_sq, d_sk, d_sv};
  const int64_t n3[3] = {Nq, Nk, Nv};
  for (int p = 0; p < 3; ++p) {
    if (n3[p] == 0) continue;
    wb[groups] = w3[p];
    yb[groups] = y3[p];
    sb[groups] = s3[p];
    nb[groups] = n3[p];
    ++groups;
  }
  // A member that fp8_linear would run with K split over two wave groups is
  // launched on its own, so that every output equals fp8_linear's bit for bit.
  bool split = false;
  for (int p = 0; p < groups; ++p) split = split || gemm_splits_k(M, nb[p], H, cus, accum);
  if (e == hipSuccess && groups > 0 && !split)
    e = launch_gemm_grouped(qx, groups, wb, yb, nb, M, H, d_sx, sb, accum, cus, stream);
  for (int p = 0; p < groups && split && e == hipSuccess; ++p)
    e = launch_gemm(qx, wb[p], yb[p], M, nb[p], H, d_sx, sb[p], FP8MOT_OUT_BF16, nullptr,
                    accum, cus, stream);
  return hip_status(e);
}

static int observe_common(const uint16_t* x, const uint16_t* u, int64_t n,
                          void* d_state, int mode, float c, hipStream_t stream) {
  if (mode != FP8MOT_OBS_MAX && mode != FP8MOT_OBS_MOVING_AVG) return FP8MOT_ERR_INVALID_ARG;
  if (mode == FP8MOT_OBS_MOVING_AVG && !std::isfinite(c)) return FP8MOT_ERR_INVALID_ARG;
  if (n < 1 || x == nullptr || d_state == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(d_state) || (u != nullptr && !aligned16(u)))
    return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_observe(x, u, n, static_cast<fp8mot_observer_state_dev*>(d_state),
                                   mode, c, ew_blocks(cus), stream));
}

int fp8_observe(const uint16_t* x, int64_t n, void* d_state, int mode, float c,
                hipStream_t stream) {
  return observe_common(x, nullptr, n, d_state, mode, c, stream);
}

int fp8_observe_swiglu(const uint16_t* g, const uint16_t* u, int64_t n,
                       void* d_state, int mode, float c, hipStream_t stream) {
  if (u == nullptr) return FP8MOT_ERR_INVALID_ARG;
  return observe_common(g, u, n, d_state, mode, c, stream);
}

int fp8_scale_from_state(const void* d_state, float* d_scale, hipStream_t stream) {
  if (d_state == nullptr || d_scale == nullptr) return FP8MOT_ERR_INVALID_ARG;
  if (!aligned16(d_state)) return FP8MOT_ERR_MISALIGNED;
  int cus = 0;
  int st = current_device(&cus);
  if (st != FP8MOT_OK) return st;
  return hip_status(launch_scale_from_state(
      static_cast<const fp8mot_observer_state_dev*>(d_state), d_scale, stream));
}

int fp8_check_shared_scale(const float* h_scales, int n) {
  if (h_scales == nullptr || n < 1) return FP8MOT_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!std::isfinite(h_scales[i]) || !(h_scales[i] > 0.0f)) return FP8MOT_ERR_INVALID_ARG;
  uint32_t b0;
  std::memcpy(&b0, &h_scales[0], 4);
  for (int i = 1; i < n; ++i) {
    uint32_t b;
    std::memcpy(&b, &h_scales[i], 4);
    if (b != b0) return FP8MOT_ERR_SCALE_MISMATCH;
  }
  return FP8MOT_OK;
}

}  // extern "C"

static_assert(sizeof(fp8mot_observer_state) == 16, "observer state is 16 bytes");
static_assert(sizeof(fp8mot_observer_state_dev) == sizeof(fp8mot_observer_state),
              "device and public observer state agree");
