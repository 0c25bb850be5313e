"""Static per-tensor FP8 (OCP E4M3FN) W8A8 Linear stack for AMD MI355X.

The compute lives in ``libfp8mot.so`` (HIP kernels for gfx950 behind a C
ABI, declared in ``include/fp8mot.h``); ``mlp_fp8_quant_amd.api`` is the thin
PyTorch binding with the same names.  The library is loaded on first use and
its absence is an error -- there is no CPU path.
"""

from .api import (ACC_EXACT, ACC_FP8_MFMA, CONV_BF16, CONV_E4M3_INT,  # noqa: F401
                  CONV_E4M3_PACKED, OBS_MAX,
                  OBS_MOVING_AVG, OUT_BF16, OUT_F32,
                  OUT_FP8, Fp8motError, debug_quant_launches,
                  convert_f32, fp8_check_shared_scale, fp8_gate_up_swiglu, fp8_linear,
                  fp8_linear_into, fp8_linear_rowwise, fp8_quant_per_row,
                  fp8_requantize_onto_max,
                  fp8_observe,
                  fp8_observe_swiglu, fp8_quant_static, fp8_scale_from_state,
                  gated_mlp_fp8, gated_mlp_fp8_noalloc, gated_mlp_fp8_workspace, init,
                  mfma_ceiling,
                  new_observer_state, qkv_fp8, qkv_fp8_workspace, rtn_weight, rw_ceiling,
                  silu_mul_2in_fp8, silu_mul_fp8)
