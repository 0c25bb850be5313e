"""PyTorch-facing binding of libfp8mot: same names as the C ABI.

Torch provides device memory and the current stream; every computation runs
in libfp8mot's HIP kernels.  Each wrapper checks dtype, device and
contiguity and refuses anything else (a strided tensor is rejected, never
copied), flattens rank-N ``[..., H]`` activations to ``[M, H]``, and maps a
non-OK status to ``Fp8motError``.

Dtypes at this boundary: BF16 tensors are ``torch.bfloat16``; FP8 tensors
are ``torch.uint8`` holding E4M3FN codes; scales are one-element
``torch.float32`` device tensors.
"""

import ctypes
import math

import torch

from . import _lib
from ._lib import Fp8motError  # noqa: F401

OUT_BF16, OUT_FP8, OUT_F32 = 0, 1, 2
ACC_EXACT, ACC_FP8_MFMA = 0, 1
OBS_MAX, OBS_MOVING_AVG = 0, 1
CONV_E4M3_PACKED, CONV_E4M3_INT, CONV_BF16 = 0, 1, 2
_OUT_DTYPE = {OUT_BF16: torch.bfloat16, OUT_FP8: torch.uint8, OUT_F32: torch.float32}


# Host cost per call matters for the small, latency-bound launches: the raw
# handle of the device's current stream (the capture stream under graph
# capture) is taken without building a Stream object, and pointers go to
# ctypes as plain integers (None for NULL).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_get_device = getattr(torch._C, "_cuda_getDevice", torch.cuda.current_device)


def _stream(t):
    # the library works on the current HIP device (its CU count and
    # architecture check come from there): tensors on another device are
    # refused rather than launched on a stream of the wrong device
    d = t.get_device()
    if d != _get_device():
        raise ValueError(f"tensors are on cuda:{d} but the current device is "
                         f"cuda:{_get_device()}; call under torch.cuda.device({d})")
    if _raw_stream is not None:
        return _raw_stream(d)
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _need(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (strided tensors are refused)")


def _scale(t, name, device):
    if t is None:
        return None  # the library refuses a NULL scale (dynamic quantization)
    _need(t, name, torch.float32, device)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold exactly one float32")
    return t


def fp8_quant_static(x, scale, out=None):
    """E4M3 codes of BF16 ``x`` at the static per-tensor ``scale``."""
    _need(x, "x", torch.bfloat16)
    _scale(scale, "scale", x.device)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, "out", torch.uint8, x.device)
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _lib.call("fp8_quant_static", _ptr(x), _ptr(out), x.numel(), _ptr(scale),
              _stream(x))
    return out


def fp8_linear(qx, qw, sx, sw, out_kind=OUT_BF16, sy=None, out=None,
               accum=ACC_EXACT):
    """y = (qx . qw^T) * (sx * sw) with qx [..., K] and qw [N, K] E4M3.

    ``accum``: ACC_EXACT (F16 matrix cores on exactly decoded codes, FP32-grade
    accumulation) or ACC_FP8_MFMA (native FP8 matrix cores, 2x the rate, with
    the hardware's 8-product windowed accumulation)."""
    _need(qx, "qx", torch.uint8)
    _need(qw, "qw", torch.uint8, qx.device)
    if qw.dim() != 2 or qx.dim() < 1 or qx.shape[-1] != qw.shape[1]:
        raise ValueError("shapes: qx [..., K], qw [N, K]")
    _scale(sx, "sx", qx.device)
    _scale(sw, "sw", qx.device)
    _scale(sy, "sy", qx.device)
    K = qw.shape[1]
    N = qw.shape[0]
    M = math.prod(qx.shape[:-1])
    if out is None:
        out = torch.empty((*qx.shape[:-1], N), dtype=_OUT_DTYPE[out_kind],
                          device=qx.device)
    _need(out, "out", _OUT_DTYPE[out_kind], qx.device)
    if out.numel() != M * N:
        raise ValueError("out must hold M * N elements")
    _lib.call("fp8_linear", _ptr(qx), _ptr(qw), _ptr(out), M, N, K, _ptr(sx),
              _ptr(sw), out_kind, _ptr(sy), accum, _stream(qx))
    return out


def fp8_quant_per_row(x, out=None, scales=None):
    """Per-row dynamic FP8 quantization of a BF16 [..., K] tensor (K % 16 ==
    0): returns (codes [..., K], FP32 scales [...]) with scale = amax(row) /
    448 and codes = e4m3(x / scale) -- per-token activations, or per-channel
    weights at load."""
    _need(x, "x", torch.bfloat16)
    if x.dim() == 0:
        raise ValueError("x must have a last (K) dimension")
    K = x.shape[-1]
    rows = math.prod(x.shape[:-1])
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _need(out, "out", torch.uint8, x.device)
    _need(scales, "scales", torch.float32, x.device)
    if out.numel() != x.numel() or scales.numel() != rows:
        raise ValueError("out must match x and scales must hold one value per row")
    _lib.call("fp8_quant_per_row", _ptr(x), _ptr(out), _ptr(scales), rows, K,
              _stream(x))
    return out, scales


def fp8_linear_rowwise(qx, qw, sx, sw, out_kind=OUT_BF16, out=None, accum=ACC_EXACT):
    """y[m, n] = acc * fp32(sx[m] * sw[n]) with acc = sum_k dec(qx) dec(qw);
    qx [..., K] E4M3 with per-row scales sx [...] (FP32), qw [N, K] with
    per-channel scales sw [N].  out_kind OUT_BF16 or OUT_F32."""
    _need(qx, "qx", torch.uint8)
    dev = qx.device
    _need(qw, "qw", torch.uint8, dev)
    K = qx.shape[-1]
    N = qw.shape[0]
    if qw.dim() != 2 or qw.shape[1] != K:
        raise ValueError("qw must be [N, K] with qx [..., K]")
    M = math.prod(qx.shape[:-1])
    _need(sx, "sx", torch.float32, dev)
    _need(sw, "sw", torch.float32, dev)
    if sx.numel() != M or sw.numel() != N:
        raise ValueError("sx must hold one scale per row of qx and sw one per row of qw")
    dtype = {OUT_BF16: torch.bfloat16, OUT_F32: torch.float32}.get(out_kind)
    if dtype is None:
        raise ValueError("out_kind must be OUT_BF16 or OUT_F32")
    if out is None:
        out = torch.empty((*qx.shape[:-1], N), dtype=dtype, device=dev)
    _need(out, "out", dtype, dev)
    if out.numel() != M * N:
        raise ValueError("out must hold M * N elements")
    _lib.call("fp8_linear_rowwise", _ptr(qx), _ptr(qw), _ptr(out), M, N, K,
              _ptr(sx), _ptr(sw), out_kind, accum, _stream(qx))
    return out


def fp8_linear_into(qx, qw, sx, sw, out, col0=0, out_kind=OUT_BF16, sy=None,
                    accum=ACC_EXACT):
    """fp8_linear writing into columns [col0, col0 + N) of an existing
    row-major output ``out`` [..., L] (L >= col0 + N): the row stride of the
    written block is L.  Nothing outside that column block is touched."""
    _need(qx, "qx", torch.uint8)
    dev = qx.device
    _need(qw, "qw", torch.uint8, dev)
    K = qx.shape[-1]
    N = qw.shape[0]
    if qw.dim() != 2 or qw.shape[1] != K:
        raise ValueError("qw must be [N, K] with qx [..., K]")
    M = math.prod(qx.shape[:-1])
    _scale(sx, "sx", dev)
    _scale(sw, "sw", dev)
    dtype = {OUT_BF16: torch.bfloat16, OUT_FP8: torch.uint8, OUT_F32: torch.float32}[out_kind]
    _need(out, "out", dtype, dev)
    L = out.shape[-1]
    if out.numel() != M * L or col0 < 0 or col0 + N > L:
        raise ValueError("out must be [..., L] with M rows and col0 + N <= L")
    if out_kind == OUT_FP8:
        _scale(sy, "sy", dev)
    base = out.data_ptr() + col0 * out.element_size()
    _lib.call("fp8_linear_ldc", _ptr(qx), _ptr(qw), ctypes.c_void_p(base), M, N, K, L,
              _ptr(sx), _ptr(sw), out_kind, _ptr(sy) if sy is not None else None,
              accum, _stream(qx))
    return out


def fp8_requantize_onto_max(qw, s_member, s_group, out=None):
    """Codes of qw re-quantized onto the largest scale of its group (the fused
    single-scale failure mode; comparison workloads only)."""
    _need(qw, "qw", torch.uint8)
    dev = qw.device
    _scale(s_member, "s_member", dev)
    _need(s_group, "s_group", torch.float32, dev)
    if out is None:
        out = torch.empty_like(qw)
    _need(out, "out", torch.uint8, dev)
    if out.numel() != qw.numel():
        raise ValueError("out must match qw")
    _lib.call("fp8_requantize_onto_max", _ptr(qw), _ptr(out), qw.numel(), _ptr(s_member),
              _ptr(s_group), s_group.numel(), _stream(qw))
    return out


def silu_mul_2in_fp8(g, u, s_out, out=None, alpha=None, beta=None):
    """E4M3 codes of g * sigmoid(alpha g) * (u + beta) at ``s_out``; g and u
    BF16 of equal shape.  Without alpha and beta this is plain SwiGLU
    (silu(g) * u); alpha is a gain inside the sigmoid, beta an offset on up."""
    _need(g, "g", torch.bfloat16)
    _need(u, "u", torch.bfloat16, g.device)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    _scale(s_out, "s_out", g.device)
    if out is None:
        out = torch.empty(g.shape, dtype=torch.uint8, device=g.device)
    _need(out, "out", torch.uint8, g.device)
    if out.numel() != g.numel():
        raise ValueError("out must have as many elements as g")
    if alpha is None and beta is None:
        _lib.call("silu_mul_2in_fp8", _ptr(g), _ptr(u), _ptr(out), g.numel(),
                  _ptr(s_out), _stream(g))
    else:
        _lib.call("silu_mul_2in_fp8_ab", _ptr(g), _ptr(u), _ptr(out), g.numel(),
                  _ptr(s_out), 1.0 if alpha is None else float(alpha),
                  0.0 if beta is None else float(beta), _stream(g))
    return out


def silu_mul_fp8(x, s_out, out=None, alpha=None, beta=None):
    """One-input SwiGLU-FP8: x BF16 [..., 2I] whose rows hold the I gate values
    followed by the I up values; returns E4M3 codes [..., I] of
    g * sigmoid(alpha g) * (u + beta) at ``s_out`` (alpha 1, beta 0 when
    omitted), bit for bit what silu_mul_2in_fp8 gives on the two halves."""
    _need(x, "x", torch.bfloat16)
    if x.dim() == 0 or x.shape[-1] % 2:
        raise ValueError("x must end in an even dimension [..., 2I]")
    _scale(s_out, "s_out", x.device)
    inter = x.shape[-1] // 2
    rows = math.prod(x.shape[:-1])
    if out is None:
        out = torch.empty((*x.shape[:-1], inter), dtype=torch.uint8, device=x.device)
    _need(out, "out", torch.uint8, x.device)
    if out.numel() != rows * inter:
        raise ValueError("out must hold [..., I] elements")
    _lib.call("silu_mul_fp8", _ptr(x), _ptr(out), rows, inter, _ptr(s_out),
              1.0 if alpha is None else float(alpha),
              0.0 if beta is None else float(beta), _stream(x))
    return out


def fp8_gate_up_swiglu(qx, wg, sx, sg, wu, su, sh, out=None, accum=ACC_EXACT):
    """qh = SwiGLU-FP8 of the gate and up projections of an E4M3 activation
    qx [..., H] (wg, wu [I, H]); bitwise what fp8_linear (BF16 out) twice and
    silu_mul_2in_fp8 give when I >= H (with H > I and few tiles fp8_linear
    sums K in two halves and a code can differ by one step), in one kernel."""
    _need(qx, "qx", torch.uint8)
    dev = qx.device
    _need(wg, "wg", torch.uint8, dev)
    _need(wu, "wu", torch.uint8, dev)
    H = qx.shape[-1]
    I = wg.shape[0]
    if wg.shape != (I, H) or wu.shape != (I, H):
        raise ValueError("shapes: qx [..., H]; wg, wu [I, H]")
    for t, n in ((sx, "sx"), (sg, "sg"), (su, "su"), (sh, "sh")):
        _scale(t, n, dev)
    M = math.prod(qx.shape[:-1])
    if out is None:
        out = torch.empty((*qx.shape[:-1], I), dtype=torch.uint8, device=dev)
    _need(out, "out", torch.uint8, dev)
    if out.numel() != M * I:
        raise ValueError("out must hold M * I elements")
    _lib.call("fp8_gate_up_swiglu", _ptr(qx), _ptr(wg), _ptr(sx), _ptr(sg),
              _ptr(wu), _ptr(su), _ptr(sh), _ptr(out), M, I, H, accum, _stream(qx))
    return out


def gated_mlp_fp8_workspace(M, H, I):
    return int(_lib.lib().gated_mlp_fp8_workspace(M, H, I))


def _workspace(nbytes, device, ws):
    if ws is None:
        # 256-byte aligned: the caching allocator aligns blocks to 512 bytes
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _need(ws, "workspace", torch.uint8, device)
    return ws


def gated_mlp_fp8(x, sx, wg, sg, wu, su, sh, wd, sd, out=None, workspace=None,
                  accum=ACC_EXACT):
    """Split gate/up gated MLP; x [..., H] BF16 -> y [..., H] BF16."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    for t, n in ((wg, "wg"), (wu, "wu"), (wd, "wd")):
        _need(t, n, torch.uint8, dev)
    H = x.shape[-1]
    I = wg.shape[0]
    if wg.shape != (I, H) or wu.shape != (I, H) or wd.shape != (H, I):
        raise ValueError("shapes: wg, wu [I, H]; wd [H, I]")
    for t, n in ((sx, "sx"), (sg, "sg"), (su, "su"), (sh, "sh"), (sd, "sd")):
        _scale(t, n, dev)
    M = math.prod(x.shape[:-1])
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if out.numel() != M * H:
        raise ValueError("out must hold M * H elements")
    nb = gated_mlp_fp8_workspace(M, H, I)
    ws = _workspace(nb, dev, workspace)
    _lib.call("gated_mlp_fp8", _ptr(x), M, H, I, _ptr(sx), _ptr(wg), _ptr(sg),
              _ptr(wu), _ptr(su), _ptr(sh), _ptr(wd), _ptr(sd), _ptr(out),
              _ptr(ws), ws.numel(), accum, _stream(x))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # FP8MOT_NOALLOC_SCRATCH_BYTES


def gated_mlp_fp8_noalloc(x, sx, wg, sg, wu, su, sh, wd, sd, out, accum=ACC_EXACT):
    """gated_mlp_fp8 without a workspace: the library keeps qX and qH in its
    own per-device scratch (at most NOALLOC_SCRATCH_BYTES); the caller passes
    the output.  Calls that overlap on one GPU race on that scratch."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    for t, n in ((wg, "wg"), (wu, "wu"), (wd, "wd")):
        _need(t, n, torch.uint8, dev)
    H = x.shape[-1]
    I = wg.shape[0]
    if wg.shape != (I, H) or wu.shape != (I, H) or wd.shape != (H, I):
        raise ValueError("shapes: wg, wu [I, H]; wd [H, I]")
    for t, n in ((sx, "sx"), (sg, "sg"), (su, "su"), (sh, "sh"), (sd, "sd")):
        _scale(t, n, dev)
    M = math.prod(x.shape[:-1])
    _need(out, "out", torch.bfloat16, dev)
    if out.numel() != M * H:
        raise ValueError("out must hold M * H elements")
    _lib.call("gated_mlp_fp8_noalloc", _ptr(x), M, H, I, _ptr(sx), _ptr(wg), _ptr(sg),
              _ptr(wu), _ptr(su), _ptr(sh), _ptr(wd), _ptr(sd), _ptr(out), accum,
              _stream(x))
    return out


def qkv_fp8_workspace(M, H):
    return int(_lib.lib().qkv_fp8_workspace(M, H))


def qkv_fp8(x, sx, wq, sq, wk, sk, wv, sv, outs=None, workspace=None,
            accum=ACC_EXACT):
    """Split Q/K/V over one shared quantization; returns (yq, yk, yv)."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    H = x.shape[-1]
    for t, n in ((wq, "wq"), (wk, "wk"), (wv, "wv")):
        _need(t, n, torch.uint8, dev)
        if t.dim() != 2 or t.shape[1] != H:
            raise ValueError(f"{n} must be [N, H]")
    for t, n in ((sx, "sx"), (sq, "sq"), (sk, "sk"), (sv, "sv")):
        _scale(t, n, dev)
    M = math.prod(x.shape[:-1])
    if outs is None:
        outs = tuple(torch.empty((*x.shape[:-1], w.shape[0]), dtype=torch.bfloat16,
                                 device=dev) for w in (wq, wk, wv))
    for o, w, n in zip(outs, (wq, wk, wv), ("yq", "yk", "yv")):
        _need(o, n, torch.bfloat16, dev)
        if o.numel() != M * w.shape[0]:
            raise ValueError(f"{n} must hold M * N elements")
    ws = _workspace(qkv_fp8_workspace(M, H), dev, workspace)
    yq, yk, yv = outs
    _lib.call("qkv_fp8", _ptr(x), M, H, _ptr(sx), _ptr(wq), wq.shape[0],
              _ptr(sq), _ptr(wk), wk.shape[0], _ptr(sk), _ptr(wv), wv.shape[0],
              _ptr(sv), _ptr(yq), _ptr(yk), _ptr(yv), _ptr(ws), ws.numel(),
              accum, _stream(x))
    return yq, yk, yv


def new_observer_state(device):
    """A fresh (zero-filled) 16-byte observer state on ``device``."""
    return torch.zeros(4, dtype=torch.int32, device=device)


def fp8_observe(x, state, mode=OBS_MAX, c=0.01):
    """Fold amax(|x|) of one calibration call into ``state``."""
    _need(x, "x", torch.bfloat16)
    _need(state, "state", torch.int32, x.device)
    if state.numel() != 4:
        raise ValueError("state must be a 16-byte observer state")
    _lib.call("fp8_observe", _ptr(x), x.numel(), _ptr(state), mode, c,
              _stream(x))
    return state


def fp8_observe_swiglu(g, u, state, mode=OBS_MAX, c=0.01):
    """Fold amax(|silu(g) * u|) into ``state``."""
    _need(g, "g", torch.bfloat16)
    _need(u, "u", torch.bfloat16, g.device)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    _need(state, "state", torch.int32, g.device)
    if state.numel() != 4:
        raise ValueError("state must be a 16-byte observer state")
    _lib.call("fp8_observe_swiglu", _ptr(g), _ptr(u), g.numel(), _ptr(state),
              mode, c, _stream(g))
    return state


def fp8_scale_from_state(state, out=None):
    """Static scale m / 448 from an observer state (one float32 on device)."""
    _need(state, "state", torch.int32)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=state.device)
    _need(out, "out", torch.float32, state.device)
    _lib.call("fp8_scale_from_state", _ptr(state), _ptr(out), _stream(state))
    return out


def fp8_check_shared_scale(scales):
    """Load-time check: raises Fp8motError unless all scales are equal,
    finite and > 0.  ``scales`` is a host sequence of floats."""
    n = len(scales)
    arr = (ctypes.c_float * max(n, 1))(*[float(s) for s in scales])
    _lib.call("fp8_check_shared_scale", arr, n)


def rw_ceiling(a, b, out):
    """Measurement aid: the quantize (b None) or SwiGLU (b given) byte mix with
    no arithmetic; out[i] = low byte of a[i] (^ b[i]).  a, b: 16-bit tensors
    (any 2-byte dtype), out: uint8 with as many elements."""
    if a.element_size() != 2 or (b is not None and b.element_size() != 2):
        raise ValueError("a and b must hold 2-byte elements")
    for t, n in ((a, "a"), (out, "out")) + (((b, "b"),) if b is not None else ()):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous GPU tensor")
    if out.dtype != torch.uint8 or out.numel() != a.numel() or (
            b is not None and b.numel() != a.numel()):
        raise ValueError("out must be uint8 with as many elements as a (and b)")
    _lib.call("fp8mot_rw_ceiling", _ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(a))
    return out


def mfma_ceiling(a, b, iters, sink, accum=ACC_EXACT):
    """Measurement aid: 8 * iters dense MFMAs per wave on fragments built from
    the E4M3 codes in a and b (uint8 GPU tensors, indices wrapped), with
    nothing else in the loop; accum selects the F16 (exact engine) or the
    native FP8 instruction.  sink: one float32 GPU element, written only if
    the products sum to a sentinel.  Returns the launch's FLOP count."""
    _need(a, "a", torch.uint8)
    _need(b, "b", torch.uint8, a.device)
    _need(sink, "sink", torch.float32, a.device)
    flops = ctypes.c_double(0.0)
    _lib.call("fp8mot_mfma_ceiling", _ptr(a), a.numel(), _ptr(b), b.numel(), int(iters),
              int(accum), _ptr(sink), ctypes.byref(flops), _stream(a))
    return flops.value


def convert_f32(x, kind=CONV_E4M3_PACKED, out=None):
    """Verification aid: the kernels' FP32 -> E4M3 (kind CONV_E4M3_PACKED or
    CONV_E4M3_INT; uint8 codes) or FP32 -> BF16 (CONV_BF16; bfloat16 bits)
    conversion of every element of the float32 GPU tensor x (numel a
    multiple of 4).  Returns out (allocated when None)."""
    _need(x, "x", torch.float32)
    dtype = torch.bfloat16 if kind == CONV_BF16 else torch.uint8
    if out is None:
        out = torch.empty(x.shape, dtype=dtype, device=x.device)
    else:
        _need(out, "out", dtype, x.device)
        if out.numel() != x.numel():
            raise ValueError("out must have as many elements as x")
    _lib.call("fp8mot_convert_f32", _ptr(x), _ptr(out), x.numel(), int(kind), _stream(x))
    return out


def debug_quant_launches():
    return int(_lib.lib().fp8mot_debug_quant_launches())


def init(device=0):
    _lib.call("fp8mot_init", int(device))


def rtn_weight(w, state=None):
    """RTN per-tensor E4M3 weight with scale amax/448, on the GPU:
    fp8_observe (max) -> fp8_scale_from_state -> fp8_quant_static."""
    st = new_observer_state(w.device)
    fp8_observe(w, st, OBS_MAX)
    s = fp8_scale_from_state(st)
    return fp8_quant_static(w, s), s
