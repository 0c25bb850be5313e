/* A plain C caller of libfp8mot (include/fp8mot.h), with no Python or torch
 * in between: it owns its device buffers (hipMalloc), passes plain pointers,
 * sizes and a stream, and checks every status.  Used by
 * tests/test_gpu_capi_consumer.py, which writes the inputs and checks the
 * outputs.
 *
 *   capi_consumer IN OUT
 *
 * IN:  int64 M, H, I; BF16 bits x [M, H]; E4M3 codes wg [I, H], wu [I, H],
 *      wd [H, I]; float32 sx, sg, su, sh, sd.
 * OUT: qx = fp8_quant_static(x; sx) [M, H] codes; G = fp8_linear(qx, wg)
 *      [M, I] BF16; y = gated_mlp_fp8(x, ...) [M, H] BF16; then int32 status
 *      of one refused call (a NULL scale: dynamic quantization).
 * Exit status 0 when every call returned FP8MOT_OK; otherwise the failing
 * call is named on stderr and the status is the exit code. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fp8mot.h"

static int fail(const char* what, int st) {
  fprintf(stderr, "%s: status %d (%s)\n", what, st, fp8mot_status_string(st));
  return st ? st : 1;
}

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static void* read_exact(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  if (!hip_ok(hipMalloc(&d, bytes ? bytes : 1), "hipMalloc")) return NULL;
  if (!hip_ok(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device")) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("open input", 0);
  int64_t dims[3];
  if (fread(dims, sizeof dims, 1, in) != 1) return fail("read sizes", 0);
  const int64_t M = dims[0], H = dims[1], I = dims[2];
  if (M <= 0 || H <= 0 || I <= 0 || M > 65536 || H > 65536 || I > 65536) return fail("sizes", 0);
  const size_t mh = (size_t)(M * H), ih = (size_t)(I * H), mi = (size_t)(M * I);
  uint16_t* x = read_exact(in, mh * 2);
  uint8_t* wg = read_exact(in, ih);
  uint8_t* wu = read_exact(in, ih);
  uint8_t* wd = read_exact(in, ih);
  float* scales = read_exact(in, 5 * sizeof(float));
  fclose(in);
  if (!x || !wg || !wu || !wd || !scales) return fail("read input", 0);

  int st = fp8mot_init(0);
  if (st != FP8MOT_OK) return fail("fp8mot_init", st);
  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;

  uint16_t* d_x = to_device(x, mh * 2);
  uint8_t* d_wg = to_device(wg, ih);
  uint8_t* d_wu = to_device(wu, ih);
  uint8_t* d_wd = to_device(wd, ih);
  float* d_s = to_device(scales, 5 * sizeof(float));   /* sx, sg, su, sh, sd */
  uint8_t* d_qx = NULL;
  uint16_t *d_g = NULL, *d_y = NULL;
  void* d_ws = NULL;
  const size_t ws_bytes = gated_mlp_fp8_workspace(M, H, I);
  if (!d_x || !d_wg || !d_wu || !d_wd || !d_s ||
      !hip_ok(hipMalloc((void**)&d_qx, mh), "hipMalloc qx") ||
      !hip_ok(hipMalloc((void**)&d_g, mi * 2), "hipMalloc G") ||
      !hip_ok(hipMalloc((void**)&d_y, mh * 2), "hipMalloc y") ||
      !hip_ok(hipMalloc(&d_ws, ws_bytes), "hipMalloc workspace"))
    return 1;

  st = fp8_quant_static(d_x, d_qx, (int64_t)mh, d_s + 0, stream);
  if (st != FP8MOT_OK) return fail("fp8_quant_static", st);
  st = fp8_linear(d_qx, d_wg, d_g, M, I, H, d_s + 0, d_s + 1, FP8MOT_OUT_BF16, NULL,
                  FP8MOT_ACC_EXACT, stream);
  if (st != FP8MOT_OK) return fail("fp8_linear", st);
  st = gated_mlp_fp8(d_x, M, H, I, d_s + 0, d_wg, d_s + 1, d_wu, d_s + 2, d_s + 3, d_wd, d_s + 4,
                     d_y, d_ws, ws_bytes, FP8MOT_ACC_EXACT, stream);
  if (st != FP8MOT_OK) return fail("gated_mlp_fp8", st);
  /* a NULL scale asks for dynamic quantization, which the path refuses
     before launching anything */
  const int32_t refused = fp8_quant_static(d_x, d_qx, (int64_t)mh, NULL, stream);
  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

  uint8_t* qx = malloc(mh);
  uint16_t* g = malloc(mi * 2);
  uint16_t* y = malloc(mh * 2);
  if (!qx || !g || !y ||
      !hip_ok(hipMemcpy(qx, d_qx, mh, hipMemcpyDeviceToHost), "copy qx") ||
      !hip_ok(hipMemcpy(g, d_g, mi * 2, hipMemcpyDeviceToHost), "copy G") ||
      !hip_ok(hipMemcpy(y, d_y, mh * 2, hipMemcpyDeviceToHost), "copy y"))
    return 1;
  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(qx, 1, mh, out) != mh || fwrite(g, 2, mi, out) != mi ||
      fwrite(y, 2, mh, out) != mh || fwrite(&refused, sizeof refused, 1, out) != 1)
    return fail("write output", 0);
  fclose(out);

  hipFree(d_x); hipFree(d_wg); hipFree(d_wu); hipFree(d_wd); hipFree(d_s);
  hipFree(d_qx); hipFree(d_g); hipFree(d_y); hipFree(d_ws);
  hipStreamDestroy(stream);
  free(x); free(wg); free(wu); free(wd); free(scales); free(qx); free(g); free(y);
  return 0;
}
