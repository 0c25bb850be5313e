"""Two-input SwiGLU with direct FP8 emission.

Pull request "Load static FP8 Cosmos3 Nano/Super checkpoints without
re-quantizing them", section "What changed" and the first commit message: a
two-input SwiGLU computes SiLU(G) * U from two separate tensors and quantizes
the result directly for the FP8 down projection, indexing both operands as
flat contiguous runs (rank-agnostic).

Here: h = silu(g) * u in float64 with silu(g) = g / (1 + exp(-g)); then
code = enc(fp32(h / s_h)) with s_h the down projection's static input scale.

Variants (same pull request, the commit message on swiglu_alpha /
swiglu_beta, and the one on silu_and_mul needing gate and up adjacent):

* alpha is a gain inside the sigmoid and beta an offset on up:
  h = g * sigmoid(alpha * g) * (u + beta).  Reading: a zero beta is no
  offset at all (u is used as it is, so a -0 stays -0), which is what makes
  "alpha and beta omitted" identical to plain SwiGLU.
* the one-input form takes gate and up adjacent in one tensor: reading, each
  row of x [..., 2I] holds the I gate values first and then the I up values,
  and the output is [..., I].
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


def silu_mul_ab_f64(g_bf16, u_bf16, alpha=1.0, beta=0.0) -> np.ndarray:
    """h = g * sigmoid(alpha * g) * (u + beta) in float64 from BF16 inputs
    (flat); a zero beta leaves u untouched."""
    g = bf16_to_f32(g_bf16).astype(np.float64).ravel()
    u = bf16_to_f32(u_bf16).astype(np.float64).ravel()
    a = np.float64(np.float32(alpha))
    b = np.float64(np.float32(beta))
    up = u if b == 0.0 else u + b
    with np.errstate(over="ignore", invalid="ignore"):
        return g / (1.0 + np.exp(-(a * g))) * up


def silu_mul_ab_fp8(g_bf16, u_bf16, s_h, alpha=1.0, beta=0.0) -> np.ndarray:
    """E4M3 codes of g * sigmoid(alpha g) * (u + beta) at scale s_h (flat)."""
    h = silu_mul_ab_f64(g_bf16, u_bf16, alpha, beta)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = (h / np.float64(np.float32(s_h))).astype(np.float32)
    return e4m3_encode(q)


def split_adjacent(x_bf16):
    """Gate and up halves of a [..., 2I] tensor whose rows hold the I gate
    values followed by the I up values: returns (g, u), each [..., I]."""
    x = np.asarray(x_bf16)
    two_i = x.shape[-1]
    if two_i % 2:
        raise ValueError("last dimension must be even (gate and up halves)")
    i = two_i // 2
    return x[..., :i], x[..., i:]


def silu_mul_adjacent_fp8(x_bf16, s_h, alpha=1.0, beta=0.0) -> np.ndarray:
    """One-input SwiGLU-FP8: codes [..., I] from x [..., 2I]."""
    g, u = split_adjacent(x_bf16)
    codes = silu_mul_ab_fp8(g, u, s_h, alpha, beta)
    return codes.reshape(g.shape)
