"""Two-input SwiGLU with direct FP8 emission.

Pull request "Load static FP8 Cosmos3 Nano/Super checkpoints without
re-quantizing them", section "What changed" and the first commit message: a
two-input SwiGLU computes SiLU(G) * U from two separate tensors and quantizes
the result directly for the FP8 down projection, indexing both operands as
flat contiguous runs (rank-agnostic).

Here: h = silu(g) * u in float64 with silu(g) = g / (1 + exp(-g)); then
code = enc(fp32(h / s_h)) with s_h the down projection's static input scale.
"""

import numpy as np

from .formats import bf16_to_f32, e4m3_encode


def silu_mul_f64(g_bf16, u_bf16) -> np.ndarray:
    """h = g / (1 + exp(-g)) * u in float64 from BF16 inputs (flat)."""
    g = bf16_to_f32(g_bf16).astype(np.float64).ravel()
    u = bf16_to_f32(u_bf16).astype(np.float64).ravel()
    with np.errstate(over="ignore", invalid="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def silu_mul_fp8(g_bf16, u_bf16, s_h) -> np.ndarray:
    """E4M3 codes of silu(g)*u at scale s_h, flat over all elements."""
    h = silu_mul_f64(g_bf16, u_bf16)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = (h / np.float64(np.float32(s_h))).astype(np.float32)
    return e4m3_encode(q)
