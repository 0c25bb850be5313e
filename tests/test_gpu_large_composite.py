"""GPU parity of the gated-MLP composite at the large compute-bound size
(X [16384, 5120], gate/up [25600, 5120], down [5120, 25600]) in the launch
configuration the benchmark times, on seeded samples the oracle computes one
by one:

* RTN weights: every sampled weight row's codes and each tensor's scale equal
  the oracle's (the oracle quantizes only the sampled rows, with the scale of
  the whole tensor);
* the fused gate/up + SwiGLU-FP8 kernel: 32 sampled token rows x 256 sampled
  intermediate columns against the oracle chain (exact sums, BF16 epilogue,
  SwiGLU, encode) -- at most one E4M3 step on at most 0.1% of them;
* gated_mlp_fp8 equals its parts (fused kernel, then fp8_linear) bit for bit;
* the down projection's shape [16384, 5120] x [5120, 25600]^T with random
  codes: 32 sampled rows x 64 sampled columns against the exact sum.
The down scale s_h is the oracle's amax/448 of silu(G)*U over the sampled
outputs (any positive scale serves parity; this one keeps codes in range)."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin
from oracle.swiglu import silu_mul_f64, silu_mul_fp8

from gpu_util import (check_fp8_tolerance, check_gemm_bf16, check_gemm_f32, device,
                      host_bits, host_f32, host_u8, oracle_rtn_threaded, scalar, to_dev_bf16,
                      to_dev_u8)

pytestmark = pytest.mark.gpu

M, H, I = 16384, 5120, 25600


def test_large_gated_mlp_composite_sampled():
    dev = device()
    wl = workloads.gated_mlp(0, M, H, I, std=0.015)
    smp = np.random.default_rng(11)
    rows = np.sort(smp.choice(M, 32, replace=False))
    cols = np.sort(smp.choice(I, 256, replace=False))
    # weights: RTN on the GPU, sampled rows checked against the oracle
    dq, ds, oq, os_ = {}, {}, {}, {}
    for k, w in wl.weights.items():
        dq[k], ds[k] = fp8.rtn_weight(to_dev_bf16(w, dev))
        os_[k] = olin.scale_from_amax(olin.amax_f32(w))
        assert ds[k].item() == float(os_[k]), k
    for k in ("gate", "up"):
        oq[k] = olin.quant_static(wl.weights[k][cols], os_[k])
        assert np.array_equal(host_u8(dq[k][torch.from_numpy(cols).to(dev)]), oq[k]), k
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    qx_rows = olin.quant_static(wl.x[rows], sx)
    Sg, Ag = olin.gemm_exact(qx_rows, oq["gate"])
    Su, Au = olin.gemm_exact(qx_rows, oq["up"])
    G = olin.epilogue_bf16(Sg, sx, os_["gate"])
    U = olin.epilogue_bf16(Su, sx, os_["up"])
    sh = olin.scale_from_amax(np.float32(np.max(np.abs(silu_mul_f64(G, U)))))
    want = silu_mul_fp8(G, U, sh).reshape(rows.size, cols.size)
    # GPU: the composite and its parts
    dx = to_dev_bf16(wl.x, dev)
    dsx, dsh = scalar(sx, dev), scalar(sh, dev)
    y = fp8.gated_mlp_fp8(dx, dsx, dq["gate"], ds["gate"], dq["up"], ds["up"], dsh,
                          dq["down"], ds["down"])
    qx = fp8.fp8_quant_static(dx, dsx)
    qh = fp8.fp8_gate_up_swiglu(qx, dq["gate"], dsx, ds["gate"], dq["up"], ds["up"], dsh)
    y2 = fp8.fp8_linear(qh, dq["down"], dsh, ds["down"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert np.array_equal(host_u8(qx[torch.from_numpy(rows).to(dev)]), qx_rows)
    got = host_u8(qh[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)])
    check_fp8_tolerance(got.ravel(), want.ravel())


def test_large_down_shape_random_codes_sampled():
    dev = device()
    rng = np.random.default_rng(12)
    qa = rng.integers(0, 256, (M, I), dtype=np.int64).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E
    qb = rng.integers(0, 256, (H, I), dtype=np.int64).astype(np.uint8)
    qb[(qb & 0x7F) == 0x7F] = 0x7E
    sx, sw = np.float32(0.0213), np.float32(1.7e-4)
    dsx, dsw = scalar(sx, dev), scalar(sw, dev)
    da, db = to_dev_u8(qa, dev), to_dev_u8(qb, dev)
    y32 = fp8.fp8_linear(da, db, dsx, dsw, fp8.OUT_F32)
    yb = fp8.fp8_linear(da, db, dsx, dsw, fp8.OUT_BF16)
    torch.cuda.synchronize()
    smp = np.random.default_rng(13)
    rows = np.sort(smp.choice(M, 32, replace=False))
    cols = np.sort(smp.choice(H, 64, replace=False))
    S, A = olin.gemm_exact(qa[rows], qb[cols])
    alpha = olin.epilogue_alpha(sx, sw)
    r, c = torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)
    f = host_f32(y32[r][:, c])
    check_gemm_f32(f, S, A, alpha)
    check_gemm_bf16(host_bits(yb[r][:, c]), f, S, A, alpha)


def test_large_gated_mlp_sampled_rows_through_the_whole_chain():
    # 16 token rows of the large gated MLP through every stage at full width,
    # each oracle stage consuming the GPU's previous-stage output: all codes
    # of the three RTN weights; qX of the rows; all 25600 SwiGLU codes of each
    # row against the oracle's chain (exact sums, BF16 epilogue, SwiGLU,
    # encode) within the SwiGLU bar; the down projection of the GPU's qH rows
    # against the exact sum (FP32 output of the same kernel within
    # 1e-5 * sum|terms|, the composite's BF16 output per R-13)
    dev = device()
    wl = workloads.gated_mlp(0, M, H, I, std=0.015)
    rows = np.sort(np.random.default_rng(14).choice(M, 16, replace=False))
    r = torch.from_numpy(rows).to(dev)
    dq, ds, oq, os_ = {}, {}, {}, {}
    for k, w in wl.weights.items():
        print(f"RTN {k} {w.shape}", flush=True)
        dq[k], ds[k] = fp8.rtn_weight(to_dev_bf16(w, dev))
        oq[k], os_[k] = oracle_rtn_threaded(w)
        assert ds[k].item() == float(os_[k]), k
        assert np.array_equal(host_u8(dq[k]), oq[k]), k
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    qx_rows = olin.quant_static(wl.x[rows], sx)
    Sg, _ = olin.gemm_exact(qx_rows, oq["gate"])
    Su, _ = olin.gemm_exact(qx_rows, oq["up"])
    G = olin.epilogue_bf16(Sg, sx, os_["gate"])
    U = olin.epilogue_bf16(Su, sx, os_["up"])
    sh = olin.scale_from_amax(np.float32(np.max(np.abs(silu_mul_f64(G, U)))))
    dx = to_dev_bf16(wl.x, dev)
    dsx, dsh = scalar(sx, dev), scalar(sh, dev)
    y = fp8.gated_mlp_fp8(dx, dsx, dq["gate"], ds["gate"], dq["up"], ds["up"], dsh,
                          dq["down"], ds["down"])
    qx = fp8.fp8_quant_static(dx, dsx)
    qh = fp8.fp8_gate_up_swiglu(qx, dq["gate"], dsx, ds["gate"], dq["up"], ds["up"], dsh)
    y32 = fp8.fp8_linear(qh, dq["down"], dsh, ds["down"], fp8.OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(qx[r]), qx_rows)
    qh_rows = host_u8(qh[r])
    check_fp8_tolerance(qh_rows.ravel(), silu_mul_fp8(G, U, sh))
    S, A = olin.gemm_exact(qh_rows, oq["down"])
    alpha = olin.epilogue_alpha(sh, os_["down"])
    f = host_f32(y32[r])
    check_gemm_f32(f, S, A, alpha)
    check_gemm_bf16(host_bits(y[r]), f, S, A, alpha)
