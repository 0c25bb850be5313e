"""GPU check of the C ABI from a plain C caller (tests/host/capi_consumer.c,
built by __graft_entry__.build()): with no Python or torch between the caller
and the library, its quantized activation is the oracle's bit for bit, its
gate projection meets the GEMM bar against the oracle's exact sum, its gate
projection and gated MLP output are bitwise what the Python binding gives on
the same inputs, and a NULL scale is refused with FP8MOT_ERR_UNSUPPORTED."""

import os
import subprocess

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin
from oracle.swiglu import silu_mul_f64

from gpu_util import (check_gemm_bf16, check_gemm_f32, device, host_bits, scalar,
                      to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "capi_consumer")


def test_c_caller_matches_oracle_and_binding(tmp_path):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build()")
    dev = device()
    M, H, I = 200, 512, 1024
    wl = workloads.gated_mlp(5, M, H, I)
    q, s = {}, {}
    for k, w in wl.weights.items():
        q[k], s[k] = olin.rtn_weight(w)
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    qx = olin.quant_static(wl.x, sx)
    Sg, Ag = olin.gemm_exact(qx, q["gate"])
    Su, _ = olin.gemm_exact(qx, q["up"])
    G = olin.epilogue_bf16(Sg, sx, s["gate"])
    U = olin.epilogue_bf16(Su, sx, s["up"])
    sh = olin.scale_from_amax(np.float32(np.max(np.abs(silu_mul_f64(G, U)))))
    scales = np.array([sx, s["gate"], s["up"], sh, s["down"]], np.float32)

    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(np.array([M, H, I], np.int64).tobytes())
        f.write(np.ascontiguousarray(wl.x, np.uint16).tobytes())
        for k in ("gate", "up", "down"):
            f.write(np.ascontiguousarray(q[k], np.uint8).tobytes())
        f.write(scales.tobytes())
    print(f"running {EXE} M={M} H={H} I={I}", flush=True)
    r = subprocess.run([EXE, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(fout, "rb").read()
    c_qx = np.frombuffer(raw, np.uint8, M * H, 0).reshape(M, H)
    c_g = np.frombuffer(raw, np.uint16, M * I, M * H).reshape(M, I)
    c_y = np.frombuffer(raw, np.uint16, M * H, M * H + 2 * M * I).reshape(M, H)
    refused = int(np.frombuffer(raw, np.int32, 1, M * H + 2 * M * I + 2 * M * H)[0])

    assert np.array_equal(c_qx, qx)
    alpha = olin.epilogue_alpha(sx, s["gate"])
    # the BF16 gate output against the exact sum (the FP32 output comes from
    # the binding's launch of the same kernel on the same operands)
    dqx, dwg = to_dev_u8(qx, dev), to_dev_u8(q["gate"], dev)
    dsx, dsg = scalar(sx, dev), scalar(s["gate"], dev)
    y32 = fp8.fp8_linear(dqx, dwg, dsx, dsg, fp8.OUT_F32).cpu().numpy()
    check_gemm_f32(y32, Sg, Ag, alpha)
    check_gemm_bf16(c_g, y32, Sg, Ag, alpha)
    assert np.array_equal(c_g, host_bits(fp8.fp8_linear(dqx, dwg, dsx, dsg)))

    dw = {k: to_dev_u8(v, dev) for k, v in q.items()}
    y = fp8.gated_mlp_fp8(to_dev_bf16(wl.x, dev), dsx, dw["gate"], dsg, dw["up"],
                          scalar(s["up"], dev), scalar(sh, dev), dw["down"], scalar(s["down"], dev))
    torch.cuda.synchronize()
    assert np.array_equal(c_y, host_bits(y))
    assert refused == 4   # FP8MOT_ERR_UNSUPPORTED
