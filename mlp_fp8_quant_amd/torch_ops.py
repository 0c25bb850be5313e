"""The libfp8mot calls as PyTorch custom operators (namespace ``fp8mot``).

Pull request "Load static FP8 Cosmos3 Nano/Super checkpoints without
re-quantizing them", first commit message: the two-input SwiGLU carries the
full custom-op contract -- a fake (shape) kernel, opcheck,
torch.compile(fullgraph=True) and graph capture.  Here every hot-path call
is registered with ``torch.library.custom_op``: the real kernel is the
libfp8mot entry point (through ``mlp_fp8_quant_amd.api``), and a fake kernel
states the output shapes and dtypes so that tracing (FakeTensor, dynamo with
fullgraph) never runs the library.  The ops allocate their outputs and
workspaces with torch, launch on the current stream and never synchronize, so
they can be captured in a HIP graph.

Scales are 1-element FP32 device tensors; weights are E4M3 codes (uint8).
"""

import math

import torch

from . import api

NS = "fp8mot"


def _rows(t):
    return math.prod(t.shape[:-1])


@torch.library.custom_op(f"{NS}::quant_static", mutates_args=())
def quant_static(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """E4M3 codes of BF16 x at the static per-tensor scale."""
    return api.fp8_quant_static(x, scale)


@quant_static.register_fake
def _(x, scale):
    return torch.empty(x.shape, dtype=torch.uint8, device=x.device)


@torch.library.custom_op(f"{NS}::linear", mutates_args=())
def linear(qx: torch.Tensor, qw: torch.Tensor, sx: torch.Tensor, sw: torch.Tensor,
           accum: int = api.ACC_EXACT) -> torch.Tensor:
    """BF16 y = (qx . qw^T) * (sx * sw)."""
    return api.fp8_linear(qx, qw, sx, sw, accum=accum)


@linear.register_fake
def _(qx, qw, sx, sw, accum=api.ACC_EXACT):
    return torch.empty((*qx.shape[:-1], qw.shape[0]), dtype=torch.bfloat16, device=qx.device)


@torch.library.custom_op(f"{NS}::silu_mul_2in", mutates_args=())
def silu_mul_2in(g: torch.Tensor, u: torch.Tensor, s_out: torch.Tensor,
                 alpha: float = 1.0, beta: float = 0.0) -> torch.Tensor:
    """E4M3 codes of g * sigmoid(alpha g) * (u + beta) at s_out."""
    if alpha == 1.0 and beta == 0.0:
        return api.silu_mul_2in_fp8(g, u, s_out)
    return api.silu_mul_2in_fp8(g, u, s_out, alpha=alpha, beta=beta)


@silu_mul_2in.register_fake
def _(g, u, s_out, alpha=1.0, beta=0.0):
    return torch.empty(g.shape, dtype=torch.uint8, device=g.device)


@torch.library.custom_op(f"{NS}::silu_mul", mutates_args=())
def silu_mul(x: torch.Tensor, s_out: torch.Tensor, alpha: float = 1.0,
             beta: float = 0.0) -> torch.Tensor:
    """One-input SwiGLU-FP8: x [..., 2I] (gate half, then up half) -> [..., I]."""
    return api.silu_mul_fp8(x, s_out, alpha=alpha, beta=beta)


@silu_mul.register_fake
def _(x, s_out, alpha=1.0, beta=0.0):
    return torch.empty((*x.shape[:-1], x.shape[-1] // 2), dtype=torch.uint8, device=x.device)


@torch.library.custom_op(f"{NS}::gated_mlp", mutates_args=())
def gated_mlp(x: torch.Tensor, sx: torch.Tensor, wg: torch.Tensor, sg: torch.Tensor,
              wu: torch.Tensor, su: torch.Tensor, sh: torch.Tensor, wd: torch.Tensor,
              sd: torch.Tensor, accum: int = api.ACC_EXACT) -> torch.Tensor:
    """Static FP8 gated MLP (one quantization of x, fused gate/up + SwiGLU-FP8,
    down projection) -> BF16 [..., H]."""
    return api.gated_mlp_fp8(x, sx, wg, sg, wu, su, sh, wd, sd, accum=accum)


@gated_mlp.register_fake
def _(x, sx, wg, sg, wu, su, sh, wd, sd, accum=api.ACC_EXACT):
    return torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)


@torch.library.custom_op(f"{NS}::qkv", mutates_args=())
def qkv(x: torch.Tensor, sx: torch.Tensor, wq: torch.Tensor, sq: torch.Tensor,
        wk: torch.Tensor, sk: torch.Tensor, wv: torch.Tensor, sv: torch.Tensor,
        accum: int = api.ACC_EXACT) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Split Q/K/V over one shared quantization -> three contiguous BF16 tensors."""
    return api.qkv_fp8(x, sx, wq, sq, wk, sk, wv, sv, accum=accum)


@qkv.register_fake
def _(x, sx, wq, sq, wk, sk, wv, sv, accum=api.ACC_EXACT):
    return tuple(torch.empty((*x.shape[:-1], w.shape[0]), dtype=torch.bfloat16, device=x.device)
                 for w in (wq, wk, wv))


@torch.library.custom_op(f"{NS}::quant_per_row", mutates_args=())
def quant_per_row(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-row dynamic quantization -> (codes [..., K], FP32 scales [...])."""
    return api.fp8_quant_per_row(x)


@quant_per_row.register_fake
def _(x):
    return (torch.empty(x.shape, dtype=torch.uint8, device=x.device),
            torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device))


@torch.library.custom_op(f"{NS}::linear_rowwise", mutates_args=())
def linear_rowwise(qx: torch.Tensor, qw: torch.Tensor, sx: torch.Tensor, sw: torch.Tensor,
                   accum: int = api.ACC_EXACT) -> torch.Tensor:
    """BF16 y[m, n] = acc * fp32(sx[m] * sw[n]) (per-token / per-channel scales)."""
    return api.fp8_linear_rowwise(qx, qw, sx, sw, accum=accum)


@linear_rowwise.register_fake
def _(qx, qw, sx, sw, accum=api.ACC_EXACT):
    return torch.empty((*qx.shape[:-1], qw.shape[0]), dtype=torch.bfloat16, device=qx.device)


OPS = (quant_static, linear, silu_mul_2in, silu_mul, gated_mlp, qkv, quant_per_row,
       linear_rowwise)
