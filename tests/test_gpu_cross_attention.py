"""GPU check of the cross-attention case of the split Q/K/V path (pull
request "Load static FP8 Cosmos3 Nano/Super checkpoints without re-quantizing
them", "What changed" and "Test Coverage": where k and v come from a different
tensor than q, one shared quantization must not engage).  q is projected from
the token activation X, k and v from a context tensor C, each input with its
own static scale: each distinct input is quantized exactly once (k and v
share C's codes), every projection is the oracle's chain with its own input's
scale, and the load-time shared-scale check refuses to put q's input in one
group with k/v's when their scales differ."""

import numpy as np
import pytest

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin

from gpu_util import (check_gemm_bf16, check_gemm_f32, device, host_bits, host_f32, scalar,
                      to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu


def test_cross_attention_quantizes_each_input_once_with_its_own_scale():
    dev = device()
    rng = np.random.default_rng(88)
    Mx, Mc, H, N = 384, 256, 1024, 512
    x = workloads.activations(rng, Mx, H)                       # tokens
    c = workloads.to_bf16_bits(rng.standard_normal((Mc, H)).astype(np.float32) * np.float32(7.0))
    w = {k: workloads.weights(rng, N, H, 0.02) for k in ("q", "k", "v")}
    sx = olin.scale_from_amax(olin.amax_f32(x))
    sc = olin.scale_from_amax(olin.amax_f32(c))
    assert sx != sc                                              # the two inputs' scales differ
    # load time: q's input scale and k/v's cannot form one shared group
    with pytest.raises(fp8.Fp8motError) as e:
        fp8.fp8_check_shared_scale([sx, sc, sc])
    assert e.value.status == 3                                   # FP8MOT_ERR_SCALE_MISMATCH
    fp8.fp8_check_shared_scale([sc, sc])                         # k and v share C's scale

    q, s = {}, {}
    for k, wk in w.items():
        q[k], s[k] = olin.rtn_weight(wk)
    dq = {k: to_dev_u8(v, dev) for k, v in q.items()}
    dsw = {k: scalar(v, dev) for k, v in s.items()}
    dsx, dsc = scalar(sx, dev), scalar(sc, dev)
    before = fp8.debug_quant_launches()
    qx = fp8.fp8_quant_static(to_dev_bf16(x, dev), dsx)
    qc = fp8.fp8_quant_static(to_dev_bf16(c, dev), dsc)
    outs = {"q": fp8.fp8_linear(qx, dq["q"], dsx, dsw["q"], fp8.OUT_F32),
            "k": fp8.fp8_linear(qc, dq["k"], dsc, dsw["k"], fp8.OUT_F32),
            "v": fp8.fp8_linear(qc, dq["v"], dsc, dsw["v"], fp8.OUT_F32)}
    bf = {"q": fp8.fp8_linear(qx, dq["q"], dsx, dsw["q"]),
          "k": fp8.fp8_linear(qc, dq["k"], dsc, dsw["k"]),
          "v": fp8.fp8_linear(qc, dq["v"], dsc, dsw["v"])}
    assert fp8.debug_quant_launches() - before == 2              # one per distinct input
    oqx, oqc = olin.quant_static(x, sx), olin.quant_static(c, sc)
    assert np.array_equal(qx.cpu().numpy(), oqx)
    assert np.array_equal(qc.cpu().numpy(), oqc)
    for k, (codes, s_in) in {"q": (oqx, sx), "k": (oqc, sc), "v": (oqc, sc)}.items():
        S, A = olin.gemm_exact(codes, q[k])
        alpha = olin.epilogue_alpha(s_in, s[k])
        y32 = host_f32(outs[k])
        check_gemm_f32(y32, S, A, alpha)
        check_gemm_bf16(host_bits(bf[k]), y32, S, A, alpha)
    # the wrong (shared) quantization would have been detected: C quantized
    # at X's scale gives other codes
    assert not np.array_equal(olin.quant_static(c, sx), oqc)
