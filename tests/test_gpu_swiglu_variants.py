"""GPU parity: the SwiGLU variants -- alpha (a gain inside the sigmoid), beta
(an offset on up) and the one-input kernel with gate and up adjacent in one
tensor -- against the oracle, and bit-exact against the two-input kernel
(pull request "Load static FP8 Cosmos3 Nano/Super checkpoints without
re-quantizing them": the commit messages on swiglu_alpha / swiglu_beta and on
silu_and_mul_2in)."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle.swiglu import (silu_mul_ab_f64, silu_mul_ab_fp8,
                           silu_mul_adjacent_fp8, silu_mul_fp8)

from gpu_util import (check_fp8_tolerance, device, host_u8, scalar,
                      to_dev_bf16)

pytestmark = pytest.mark.gpu

# (alpha, beta): plain, gain only, offset only, the swigluoai shape, a gain
# below one with a negative offset
CASES = [(1.0, 0.0), (1.702, 0.0), (1.0, 1.0), (1.702, 1.0), (0.5, -0.75)]


def _gu(rng, n, sg=3.0, su=2.0):
    g = workloads.to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(sg))
    u = workloads.to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(su))
    return g, u


def _scale(g, u, a, b):
    return np.float32(np.max(np.abs(silu_mul_ab_f64(g, u, a, b))) / 448)


@pytest.mark.parametrize("alpha,beta", CASES)
@pytest.mark.parametrize("n", [1, 17, 4099, 1 << 20])
def test_two_input_alpha_beta_against_oracle(alpha, beta, n):
    dev = device()
    rng = np.random.default_rng(n + int(alpha * 1000) + int(beta * 100))
    g, u = _gu(rng, n)
    s = _scale(g, u, alpha, beta)
    q = fp8.silu_mul_2in_fp8(to_dev_bf16(g, dev), to_dev_bf16(u, dev), scalar(s, dev),
                             alpha=alpha, beta=beta)
    check_fp8_tolerance(host_u8(q), silu_mul_ab_fp8(g, u, s, alpha, beta))


def test_omitting_alpha_beta_is_plain_swiglu_bitwise():
    # explicit (1, 0) through the variant entry point == the plain kernel,
    # including -0 up values (a zero beta is no offset) and the n % 16 tail
    dev = device()
    rng = np.random.default_rng(31)
    g, u = _gu(rng, 100_003)
    u[::7] = 0x8000                       # -0
    g[::11] = 0x8000
    dg, du = to_dev_bf16(g, dev), to_dev_bf16(u, dev)
    s = scalar(0.037, dev)
    plain = host_u8(fp8.silu_mul_2in_fp8(dg, du, s))
    ab = host_u8(fp8.silu_mul_2in_fp8(dg, du, s, alpha=1.0, beta=0.0))
    assert np.array_equal(plain, ab)
    # u = -0: the product is a zero whose sign is opposite to silu(g)'s
    neg0 = u == 0x8000
    assert np.count_nonzero(neg0) > 0
    assert np.array_equal(plain[neg0], silu_mul_fp8(g, u, np.float32(0.037))[neg0])


@pytest.mark.parametrize("alpha,beta", CASES)
@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (7, 13), (2, 5, 1040), (64, 8192)])
def test_one_input_bitwise_equals_two_input(alpha, beta, shape):
    # gate and up adjacent ([..., 2I], gate first) give the same codes as the
    # two-input kernel on the halves; ragged I (13) takes the scalar path
    dev = device()
    rng = np.random.default_rng(sum(shape) + int(alpha * 10))
    *lead, inter = shape
    x = workloads.to_bf16_bits(rng.standard_normal((*lead, 2 * inter)).astype(np.float32) * 3)
    s = np.float32(np.max(np.abs(silu_mul_ab_f64(x[..., :inter], x[..., inter:], alpha, beta))) / 448)
    dx = to_dev_bf16(x.ravel(), dev).view(*lead, 2 * inter)
    q1 = fp8.silu_mul_fp8(dx, scalar(s, dev), alpha=alpha, beta=beta)
    assert q1.shape == (*lead, inter)
    g = dx[..., :inter].contiguous()
    u = dx[..., inter:].contiguous()
    q2 = fp8.silu_mul_2in_fp8(g, u, scalar(s, dev), alpha=alpha, beta=beta)
    assert torch.equal(q1, q2)
    check_fp8_tolerance(host_u8(q1).ravel(), silu_mul_adjacent_fp8(x, s, alpha, beta).ravel())


def test_one_input_gen_mlp_size_against_oracle():
    # the gen-tower intermediate (M = 2048, I = 8192) as one [M, 2I] tensor
    dev = device()
    rng = np.random.default_rng(32)
    M, inter = 2048, 8192
    x = workloads.to_bf16_bits(rng.standard_normal((M, 2 * inter)).astype(np.float32) * 2)
    s = np.float32(0.02)
    q = fp8.silu_mul_fp8(to_dev_bf16(x.ravel(), dev).view(M, 2 * inter), scalar(s, dev),
                         alpha=1.702, beta=1.0)
    check_fp8_tolerance(host_u8(q).ravel(), silu_mul_adjacent_fp8(x, s, 1.702, 1.0).ravel())


def test_variant_refusals():
    dev = device()
    x = torch.zeros((4, 32), dtype=torch.bfloat16, device=dev)
    s = scalar(1.0, dev)
    with pytest.raises(ValueError):
        fp8.silu_mul_fp8(torch.zeros((4, 31), dtype=torch.bfloat16, device=dev), s)
    with pytest.raises(ValueError):
        fp8.silu_mul_fp8(x.t(), s)                       # strided: refused, not copied
    with pytest.raises(fp8.Fp8motError):
        fp8.silu_mul_fp8(x, s, alpha=float("nan"))
    with pytest.raises(fp8.Fp8motError):
        fp8.silu_mul_2in_fp8(x, x, s, beta=float("inf"))
