"""Per-row FP8: per-channel weight scales and per-token activation scales.

Model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN + moving-average activation
observer", section 3.2 (the per-channel weight / per-token activation builds)
and the paragraph after its table: the framework's runtime FP8 path with
per-row granularity quantizes the BF16 weights RTN per output channel when it
loads them, and the activations per token at run time.  The same Linear then
computes, for output (m, n),

    y[m, n] = s_x[m] * s_w[n] * sum_k dec(qx[m, k]) * dec(qw[n, k]).

Readings (the card gives the scheme, not its arithmetic):
* a row's scale is fp32(amax(row)) / 448 in FP32, as the per-tensor scale is
  for a whole tensor, and its codes are enc(fp32(x) / s_row);
* a row whose amax is 0 gets scale 0 and codes that are signed zeros
  (x / 0 is undefined; every x in the row is +-0 and keeps its sign);
* a row holding a NaN gets a NaN scale and all-NaN codes (0x7F); a row
  holding an infinity gets an infinite scale (finite elements -> +-0, the
  infinity itself -> NaN);
* the epilogue forms alpha = fp32(s_x[m] * s_w[n]) and then fp32(acc * alpha),
  as the per-tensor epilogue does with its single alpha.
"""

import numpy as np

from .formats import E4M3_MAX, bf16_to_f32, e4m3_encode, f32_to_bf16


def row_scales(x_bf16) -> np.ndarray:
    """Per-row scale fp32(amax(row)) / 448 of a BF16 [R, K] tensor (float32 [R])."""
    x = bf16_to_f32(np.asarray(x_bf16))
    if x.ndim != 2:
        raise ValueError("rows of a 2-D tensor")
    if x.shape[1] == 0:
        return np.zeros(x.shape[0], np.float32)
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(x), axis=1).astype(np.float32)
    return (amax / np.float32(E4M3_MAX)).astype(np.float32)


def quant_per_row(x_bf16):
    """(codes [R, K], scales [R]): each row quantized at its own scale."""
    xb = np.asarray(x_bf16)
    x = bf16_to_f32(xb)
    s = row_scales(xb)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        q = x / s[:, None]
    assert q.dtype == np.float32
    codes = e4m3_encode(q)
    zero = s == 0
    if np.any(zero):
        codes[zero] = ((xb[zero] >> 8) & 0x80).astype(np.uint8)   # signed zeros
    return codes, s


def rtn_weight_per_channel(w_bf16):
    """RTN per-output-channel weight: (codes [N, K], scales [N])."""
    return quant_per_row(w_bf16)


def epilogue_rowwise_alpha(sx_rows, sw_rows) -> np.ndarray:
    """alpha[m, n] = fp32(s_x[m] * s_w[n])."""
    sx = np.asarray(sx_rows, np.float32)
    sw = np.asarray(sw_rows, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return (sx[:, None] * sw[None, :]).astype(np.float32)


def epilogue_rowwise_f32(S, sx_rows, sw_rows) -> np.ndarray:
    """Pre-rounding output y32[m, n] = fp32(fp32(S[m, n]) * alpha[m, n])."""
    alpha = epilogue_rowwise_alpha(sx_rows, sw_rows)
    with np.errstate(over="ignore", invalid="ignore"):
        return (np.asarray(S).astype(np.float32) * alpha).astype(np.float32)


def epilogue_rowwise_bf16(S, sx_rows, sw_rows) -> np.ndarray:
    """BF16 output bits: RNE of the pre-rounding FP32 value."""
    return f32_to_bf16(epilogue_rowwise_f32(S, sx_rows, sw_rows))
