"""Host-only checks of the C ABI: the library loads, exports every symbol
the header declares, and refuses bad arguments before touching a device.
No kernel is launched here (no GPU in this environment)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mot.h")


def _lib():
    from mlp_fp8_quant_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libfp8mot.so is not built (run __graft_entry__.build())")
    return L.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ("fp8_quant_static", "fp8_linear", "silu_mul_2in_fp8",
              "gated_mlp_fp8", "qkv_fp8", "fp8_observe", "fp8_scale_from_state",
              "fp8_check_shared_scale", "fp8_gate_up_swiglu",
              "silu_mul_2in_fp8_ab", "silu_mul_fp8", "fp8_quant_per_row",
              "fp8_linear_rowwise", "fp8_linear_ldc", "fp8_requantize_onto_max"):
        assert n in names


def test_header_is_valid_c(tmp_path):
    # the ABI is C: the header compiles as C11 with every warning an error
    # (the ROCm headers it includes as system headers), and every declared
    # function is referenced by name from C
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.fail("gcc is required to check the header as C")
    src = tmp_path / "uses_header.c"
    refs = "\n".join(f"  (void)&{n};" for n in declared_functions())
    src.write_text('#include "fp8mot.h"\nint main(void) {\n' + refs + "\n  return 0;\n}\n")
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include",
                        "-I", os.path.dirname(HEADER), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    from mlp_fp8_quant_amd._lib import SIGNATURES
    assert set(SIGNATURES) == set(declared_functions())


def test_status_strings():
    lib = _lib()
    for st in range(8):
        assert lib.fp8mot_status_string(st) != b"unknown status"
    assert lib.fp8mot_status_string(99) == b"unknown status"


def test_check_shared_scale_host_logic():
    import mlp_fp8_quant_amd as fp8
    fp8.fp8_check_shared_scale([0.5, 0.5, 0.5])
    cases = {3: [0.5, 0.25], 1: [0.5, float("nan")]}
    for status, sc in cases.items():
        with pytest.raises(fp8.Fp8motError) as e:
            fp8.fp8_check_shared_scale(sc)
        assert e.value.status == status
    for sc in ([], [0.0, 0.0], [-1.0], [float("inf")]):
        with pytest.raises(fp8.Fp8motError) as e:
            fp8.fp8_check_shared_scale(sc)
        assert e.value.status == 1


def test_workspace_sizes():
    lib = _lib()
    M, H, I = 2048, 2048, 8192
    r = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert lib.gated_mlp_fp8_workspace(M, H, I) == r(M * H) + r(M * I)
    assert lib.qkv_fp8_workspace(3072, 4096) == 3072 * 4096
    assert lib.gated_mlp_fp8_workspace(-1, 1, 1) == 0


def test_refusals_before_any_device_access():
    lib = _lib()
    P = ctypes.c_void_p
    fake = P(0x10000)        # never dereferenced: every case below is refused
    odd = P(0x10001)         # earlier, by argument validation alone
    null = P(0)
    s = fake
    # NULL scale = dynamic quantization -> UNSUPPORTED
    assert lib.fp8_quant_static(fake, fake, 16, null, null) == 4
    assert lib.silu_mul_2in_fp8(fake, fake, fake, 16, null, null) == 4
    assert lib.fp8_linear(fake, fake, fake, 4, 4, 16, null, s, 0, null, 0, null) == 4
    assert lib.fp8_linear(fake, fake, fake, 4, 4, 16, s, s, 1, null, 0, null) == 4
    # negative sizes, K % 16, bad enums -> INVALID_ARG
    assert lib.fp8_quant_static(fake, fake, -1, s, null) == 1
    assert lib.fp8_linear(fake, fake, fake, 4, 4, 24, s, s, 0, null, 0, null) == 1
    assert lib.fp8_linear(fake, fake, fake, -4, 4, 16, s, s, 0, null, 0, null) == 1
    assert lib.fp8_linear(fake, fake, fake, 4, 4, 16, s, s, 7, null, 0, null) == 1
    assert lib.fp8_observe(fake, 16, fake, 5, ctypes.c_float(0.01), null) == 1
    assert lib.fp8_observe(fake, 0, fake, 0, ctypes.c_float(0.01), null) == 1
    assert lib.fp8_observe(fake, 16, fake, 1, ctypes.c_float(float("nan")), null) == 1
    # NULL data pointers with a non-empty size -> INVALID_ARG
    assert lib.fp8_quant_static(null, fake, 16, s, null) == 1
    # empty tensors are a valid no-op
    assert lib.fp8_quant_static(null, null, 0, s, null) == 0
    # the MFMA-ceiling measurement aid: NULL pointers, buffers under 64 codes,
    # no iterations or another engine -> INVALID_ARG
    flops = ctypes.c_double(0.0)
    fl = ctypes.byref(flops)
    assert lib.fp8mot_mfma_ceiling(null, 64, fake, 64, 1, 0, fake, fl, null) == 1
    assert lib.fp8mot_mfma_ceiling(fake, 64, fake, 64, 1, 0, null, fl, null) == 1
    assert lib.fp8mot_mfma_ceiling(fake, 64, fake, 64, 1, 0, fake, None, null) == 1
    assert lib.fp8mot_mfma_ceiling(fake, 63, fake, 64, 1, 0, fake, fl, null) == 1
    assert lib.fp8mot_mfma_ceiling(fake, 64, fake, 63, 1, 1, fake, fl, null) == 1
    assert lib.fp8mot_mfma_ceiling(fake, 64, fake, 64, 0, 0, fake, fl, null) == 1
    assert lib.fp8mot_mfma_ceiling(fake, 64, fake, 64, 1, 2, fake, fl, null) == 1
    # the conversion verification aid: n < 0 or not a multiple of 4, another
    # kind, NULL pointers -> INVALID_ARG; n == 0 is a no-op; misaligned ->
    # MISALIGNED
    assert lib.fp8mot_convert_f32(fake, fake, -4, 0, null) == 1
    assert lib.fp8mot_convert_f32(fake, fake, 6, 0, null) == 1
    assert lib.fp8mot_convert_f32(fake, fake, 8, 3, null) == 1
    assert lib.fp8mot_convert_f32(fake, fake, 8, -1, null) == 1
    assert lib.fp8mot_convert_f32(null, fake, 8, 2, null) == 1
    assert lib.fp8mot_convert_f32(fake, null, 8, 1, null) == 1
    assert lib.fp8mot_convert_f32(null, null, 0, 0, null) == 0
    assert lib.fp8mot_convert_f32(odd, fake, 8, 0, null) == 2
    assert lib.fp8mot_convert_f32(fake, odd, 8, 2, null) == 2
    assert lib.fp8_linear(null, null, null, 0, 4, 16, s, s, 0, null, 0, null) == 0
    # misaligned base pointers -> MISALIGNED
    assert lib.fp8_quant_static(odd, fake, 16, s, null) == 2
    assert lib.silu_mul_2in_fp8(fake, odd, fake, 16, s, null) == 2
    assert lib.fp8_linear(fake, fake, odd, 4, 4, 16, s, s, 0, null, 0, null) == 2
    # composites: workspace too small -> WORKSPACE
    assert lib.qkv_fp8(fake, 4, 16, s, fake, 4, s, fake, 4, s, fake, 4, s,
                       fake, fake, fake, fake, 8, 0, null) == 6
    assert lib.gated_mlp_fp8(fake, 4, 16, 32, s, fake, s, fake, s, s, fake, s,
                             fake, null, 0, 0, null) == 6
    assert lib.gated_mlp_fp8(fake, 4, 16, 32, null, fake, s, fake, s, s, fake, s,
                             fake, fake, 1 << 20, 0, null) == 4
    # I = 0: the weights are empty tensors, NULL allowed; the call gets past
    # argument validation to the workspace check
    assert lib.gated_mlp_fp8(fake, 4, 16, 0, s, null, s, null, s, s, null, s,
                             fake, null, 0, 0, null) == 6
    assert lib.gated_mlp_fp8(fake, 4, 16, 32, s, null, s, fake, s, s, fake, s,
                             fake, fake, 1 << 20, 0, null) == 1
    assert lib.fp8_gate_up_swiglu(fake, fake, s, s, fake, s, null, fake, 4, 32, 16, 0, null) == 4
    assert lib.fp8_gate_up_swiglu(fake, fake, s, s, fake, s, s, fake, 4, 24, 16, 0, null) == 1
    assert lib.fp8_gate_up_swiglu(fake, odd, s, s, fake, s, s, fake, 4, 32, 16, 0, null) == 2
    assert lib.fp8_gate_up_swiglu(null, null, s, s, null, s, s, null, 0, 32, 16, 0, null) == 0
    # sizes beyond the GEMM kernels' 32-bit tile windows -> INVALID_ARG
    # (256 rows of K codes, 256 output rows of N or ldc elements)
    kmax = 8388576                           # largest K (multiple of 16) with 256 * K < 0x7FFFF000
    assert lib.fp8_linear(null, null, null, 0, 4, kmax + 16, s, s, 0, null, 0, null) == 1
    assert lib.fp8_linear(null, null, null, 0, 4, kmax, s, s, 0, null, 0, null) == 0
    nmax_bf16 = 0x7FFFF000 // (256 * 2) - 1  # BF16 output rows
    assert lib.fp8_linear(null, null, null, 0, nmax_bf16 + 1, 16, s, s, 0, null, 0, null) == 1
    assert lib.fp8_linear(null, null, null, 0, nmax_bf16, 16, s, s, 0, null, 0, null) == 0
    # the same N fits FP8 output rows but not FP32 ones
    assert lib.fp8_linear(null, null, null, 0, nmax_bf16 + 1, 16, s, s, 1, s, 0, null) == 0
    assert lib.fp8_linear(null, null, null, 0, nmax_bf16 + 1, 16, s, s, 2, null, 0, null) == 1
    assert lib.fp8_linear_ldc(null, null, null, 0, 32, 16, nmax_bf16 + 1, s, s, 0, null, 0, null) == 1
    assert lib.fp8_gate_up_swiglu(null, null, s, s, null, s, s, null, 0, 32, kmax + 16, 0, null) == 1
    assert lib.gated_mlp_fp8(null, 0, 16, kmax + 16, s, null, s, null, s, s, null, s,
                             null, null, 0, 0, null) == 1
    assert lib.qkv_fp8(null, 0, kmax + 16, s, null, 0, s, null, 0, s, null, 0, s,
                       null, null, null, null, 0, 0, null) == 1
    assert lib.qkv_fp8(null, 0, 16, s, null, nmax_bf16 + 1, s, null, 0, s, null, 0, s,
                       null, null, null, null, 0, 0, null) == 1
    # the allocation-free gated MLP: the gated MLP's own refusals, and sizes
    # whose qX + qH exceed its fixed 64 MiB scratch -> TOO_LARGE, all before
    # any device access
    na = lib.gated_mlp_fp8_noalloc
    assert na(fake, 4, 16, 32, null, fake, s, fake, s, s, fake, s, fake, 0, null) == 4
    assert na(fake, 4, 16, 24, s, fake, s, fake, s, s, fake, s, fake, 0, null) == 1
    assert na(fake, 4, 16, 32, s, fake, s, fake, s, s, fake, s, fake, 3, null) == 1
    assert na(fake, 4, 16, 32, s, odd, s, fake, s, s, fake, s, fake, 0, null) == 2
    assert na(null, 0, 16, 32, s, null, s, null, s, s, null, s, null, 0, null) == 0
    assert na(fake, 4097, 4096, 12288, s, fake, s, fake, s, s, fake, s, fake, 0, null) == 7
    assert na(fake, 16384, 5120, 25600, s, fake, s, fake, s, s, fake, s, fake, 0, null) == 7
    assert lib.gated_mlp_fp8_workspace(4096, 4096, 12288) == 64 << 20   # fits exactly
    # unknown accumulation engine -> INVALID_ARG
    assert lib.fp8_linear(fake, fake, fake, 4, 4, 16, s, s, 0, null, 2, null) == 1
    assert lib.gated_mlp_fp8(fake, 4, 16, 32, s, fake, s, fake, s, s, fake, s,
                             fake, fake, 1 << 20, 5, null) == 1


def test_swiglu_variant_refusals_before_any_device_access():
    lib = _lib()
    P = ctypes.c_void_p
    fake = P(0x10000)        # never dereferenced: every case below is refused
    odd = P(0x10001)
    null = P(0)
    s = fake
    nan, inf = float("nan"), float("inf")
    # NULL scale -> UNSUPPORTED
    assert lib.silu_mul_2in_fp8_ab(fake, fake, fake, 16, null, 1.0, 0.0, null) == 4
    assert lib.silu_mul_fp8(fake, fake, 2, 16, null, 1.0, 0.0, null) == 4
    # non-finite alpha / beta, negative sizes -> INVALID_ARG
    assert lib.silu_mul_2in_fp8_ab(fake, fake, fake, 16, s, nan, 0.0, null) == 1
    assert lib.silu_mul_2in_fp8_ab(fake, fake, fake, 16, s, 1.0, inf, null) == 1
    assert lib.silu_mul_2in_fp8_ab(fake, fake, fake, -1, s, 1.0, 0.0, null) == 1
    assert lib.silu_mul_fp8(fake, fake, 2, 16, s, inf, 0.0, null) == 1
    assert lib.silu_mul_fp8(fake, fake, -2, 16, s, 1.0, 0.0, null) == 1
    assert lib.silu_mul_fp8(fake, fake, 2, -16, s, 1.0, 0.0, null) == 1
    assert lib.silu_mul_fp8(null, fake, 2, 16, s, 1.0, 0.0, null) == 1
    # empty -> OK without touching anything
    assert lib.silu_mul_2in_fp8_ab(null, null, null, 0, s, 1.0, 0.0, null) == 0
    assert lib.silu_mul_fp8(null, null, 0, 16, s, 1.0, 0.0, null) == 0
    assert lib.silu_mul_fp8(null, null, 3, 0, s, 1.0, 0.0, null) == 0
    # misaligned -> MISALIGNED
    assert lib.silu_mul_2in_fp8_ab(fake, odd, fake, 16, s, 1.0, 0.0, null) == 2
    assert lib.silu_mul_fp8(odd, fake, 2, 16, s, 1.0, 0.0, null) == 2
    assert lib.silu_mul_fp8(fake, odd, 2, 16, s, 1.0, 0.0, null) == 2


def test_rowwise_refusals_before_any_device_access():
    lib = _lib()
    P = ctypes.c_void_p
    fake = P(0x10000)        # never dereferenced: every case below is refused
    odd = P(0x10001)
    null = P(0)
    s = fake
    # per-row quantize: K % 16, negative sizes, NULL scales, alignment
    assert lib.fp8_quant_per_row(fake, fake, fake, 4, 24, null) == 1
    assert lib.fp8_quant_per_row(fake, fake, fake, -1, 16, null) == 1
    assert lib.fp8_quant_per_row(fake, fake, null, 4, 16, null) == 1
    assert lib.fp8_quant_per_row(odd, fake, fake, 4, 16, null) == 2
    assert lib.fp8_quant_per_row(null, null, null, 0, 16, null) == 0
    # K == 0 still writes one scale per row: the scales must be given
    assert lib.fp8_quant_per_row(null, null, null, 4, 0, null) == 1
    # per-row GEMM: FP8 output unsupported, NULL scales, bad enums, alignment
    assert lib.fp8_linear_rowwise(fake, fake, fake, 4, 4, 16, s, s, 1, 0, null) == 4
    assert lib.fp8_linear_rowwise(fake, fake, fake, 4, 4, 16, null, s, 0, 0, null) == 4
    assert lib.fp8_linear_rowwise(fake, fake, fake, 4, 4, 24, s, s, 0, 0, null) == 1
    assert lib.fp8_linear_rowwise(fake, fake, fake, 4, 4, 16, s, s, 0, 7, null) == 1
    assert lib.fp8_linear_rowwise(fake, fake, fake, 4, 4, 16, s, s, 5, 0, null) == 1
    assert lib.fp8_linear_rowwise(fake, fake, fake, 4, 4, 16, odd, s, 0, 0, null) == 2
    assert lib.fp8_linear_rowwise(null, null, null, 0, 4, 16, s, s, 0, 0, null) == 0


def test_fused_topology_refusals_before_any_device_access():
    lib = _lib()
    P = ctypes.c_void_p
    fake = P(0x10000)        # never dereferenced: every case below is refused
    odd = P(0x10001)
    null = P(0)
    s = fake
    # ldc below N, K % 16, NULL scales, alignment
    assert lib.fp8_linear_ldc(fake, fake, fake, 4, 32, 16, 31, s, s, 0, null, 0, null) == 1
    assert lib.fp8_linear_ldc(fake, fake, fake, 4, 32, 24, 64, s, s, 0, null, 0, null) == 1
    assert lib.fp8_linear_ldc(fake, fake, fake, 4, 32, 16, 64, null, s, 0, null, 0, null) == 4
    assert lib.fp8_linear_ldc(fake, fake, odd, 4, 32, 16, 64, s, s, 0, null, 0, null) == 2
    assert lib.fp8_linear_ldc(null, null, null, 0, 32, 16, 64, s, s, 0, null, 0, null) == 0
    # requantize: NULL scales, bad group size, alignment, empty
    assert lib.fp8_requantize_onto_max(fake, fake, 16, null, s, 2, null) == 4
    assert lib.fp8_requantize_onto_max(fake, fake, 16, s, null, 2, null) == 4
    assert lib.fp8_requantize_onto_max(fake, fake, 16, s, s, 0, null) == 1
    assert lib.fp8_requantize_onto_max(fake, fake, -1, s, s, 2, null) == 1
    assert lib.fp8_requantize_onto_max(odd, fake, 16, s, s, 2, null) == 2
    assert lib.fp8_requantize_onto_max(null, null, 0, s, s, 2, null) == 0
