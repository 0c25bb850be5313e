"""Static FP8 Linear: quantize, RTN weights, exact GEMM, epilogues.

Sources
-------
* Model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN ...", section "Scheme":
  weights are FP8 E4M3 with one scale per tensor (round-to-nearest, "RTN");
  activations are FP8 E4M3 with one static, calibrated scale per tensor.
* Same card, experiment setup of its fake-quant section: the fake-quant
  replay uses the dequantized FP8 weight codes together with an FP8
  quantize-dequantize of the input.  In exact arithmetic that is
  ``Y = QDQ(X; s_x) @ (s_w * dec(qW))^T = s_x * s_w * sum_k dec(qX) dec(qW)``,
  which is what the FP8 GEMM computes up to FP32 accumulation and output
  rounding; ``gemm_exact`` is that definition.
* Pull request "Load static FP8 Cosmos3 Nano/Super checkpoints without
  re-quantizing them", section "Description": a fused group that keeps one
  weight scale re-quantizes each member as FP8-round((s_i * qW_i) / max(s))
  instead of keeping s_i * qW_i.  ``requantize_onto_max`` is that failure
  mode, kept as a negative reference.
* Same pull request, commit messages: each Linear applies its own scale in
  the GEMM epilogue, so the epilogue multiplies the FP32 accumulator by
  ``s_x * s_w``.

Readings (where the pages are silent): quantization divides by the scale
(value = code * scale, so code = x / scale) with one correctly rounded FP32
division before the E4M3 rounding; the weight scale is amax / 448 in FP32;
the epilogue forms ``alpha = fp32(s_x * s_w)`` first and then
``fp32(acc * alpha)``.
"""

import numpy as np

from .formats import (E4M3_MAX, bf16_to_f32, e4m3_decode, e4m3_encode,
                      f32_to_bf16)


def quant_static(x_bf16, scale) -> np.ndarray:
    """FP8 codes of a BF16 tensor at a static per-tensor scale.

    code = enc(fp32(x) / s) with IEEE float32 division (NumPy's float32
    division is correctly rounded).
    """
    x = bf16_to_f32(x_bf16)
    s = np.float32(scale)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        q = x / s
    assert q.dtype == np.float32
    return e4m3_encode(q)


def amax_f32(x_bf16) -> np.float32:
    """max |x| of a BF16 tensor as float32 (exact); NaN if any element is NaN."""
    x = bf16_to_f32(x_bf16)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def scale_from_amax(amax) -> np.float32:
    """Per-tensor scale amax / 448 with one float32 division."""
    return np.float32(np.float32(amax) / np.float32(E4M3_MAX))


def rtn_weight(w_bf16):
    """RTN per-tensor FP8 weight: (codes, scale) with scale = amax/448."""
    s = scale_from_amax(amax_f32(w_bf16))
    return quant_static(w_bf16, s), s


def gemm_exact(qa, qb):
    """Exact S = sum_k dec(qa[m,k]) dec(qb[n,k]) and A = sum_k |same|.

    qa is [M, K] and qb is [N, K] (both K-contiguous).  Every FP8 x FP8
    product is an integer multiple of 2^-18 of magnitude <= 448^2, so each
    partial sum of K such terms is an integer multiple of 2^-18 below
    K * 448^2 * 2^18 in units; for K <= 171196 that fits in the 53-bit
    significand of float64 and the float64 matrix product is exact in any
    summation order.
    """
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    K = qa.shape[1]
    if K > 171196:
        raise ValueError("float64 accumulation is exact only for K <= 171196")
    a = e4m3_decode(qa)
    b = e4m3_decode(qb)
    S = a @ b.T
    A = np.abs(a) @ np.abs(b).T
    return S, A


def gemm_f32acc(qa, qb) -> np.ndarray:
    """FP32-accumulated product of the decoded operands (a self-check only)."""
    a = e4m3_decode(qa).astype(np.float32)
    b = e4m3_decode(qb).astype(np.float32)
    return a @ b.T


def epilogue_alpha(s_x, s_w) -> np.float32:
    """alpha = fp32(s_x * s_w)."""
    return np.float32(np.float32(s_x) * np.float32(s_w))


def epilogue_f32(S, s_x, s_w) -> np.ndarray:
    """Pre-rounding output y32 = fp32(fp32(S) * alpha)."""
    alpha = epilogue_alpha(s_x, s_w)
    with np.errstate(over="ignore"):
        return (np.asarray(S).astype(np.float32) * alpha).astype(np.float32)


def epilogue_bf16(S, s_x, s_w) -> np.ndarray:
    """BF16 output bits: RNE of the pre-rounding FP32 value."""
    return f32_to_bf16(epilogue_f32(S, s_x, s_w))


def epilogue_fp8(S, s_x, s_w, s_y) -> np.ndarray:
    """FP8 output codes: enc(fp32(y32 / s_y))."""
    y32 = epilogue_f32(S, s_x, s_w)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        return e4m3_encode(y32 / np.float32(s_y))


def requantize_onto_max(qws, scales):
    """Failure mode of a fused group holding one scale (negative reference).

    Each member i becomes enc(fp32(fp32(s_i * dec(qW_i)) / max(s))): the
    product and the quotient are each rounded once to float32.
    Returns (list of re-quantized codes, max scale).
    """
    scales = [np.float32(s) for s in scales]
    smax = np.float32(max(scales))
    out = []
    for q, s in zip(qws, scales):
        v = (e4m3_decode(q).astype(np.float32) * s).astype(np.float32)
        out.append(e4m3_encode((v / smax).astype(np.float32)))
    return out, smax


def check_shared_scale(scales) -> bool:
    """Load-time invariant of a shared-quantization group.

    Pull request section "What changed": the projections of a group must
    carry the same calibrated input_scale, validated once when the weights
    are loaded and not in the forward pass.  True iff every scale is finite,
    > 0 and all are bitwise equal.
    """
    s = np.asarray(scales, dtype=np.float32)
    if s.size == 0:
        return False
    if not np.all(np.isfinite(s)) or not np.all(s > 0):
        return False
    bits = s.view(np.uint32)
    return bool(np.all(bits == bits[0]))
