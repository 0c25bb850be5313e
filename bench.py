"""Benchmark of the static FP8 gated-MLP hot path on one MI355X.

One step = one pass of the whole path over one batch of the gen-tower gated
MLP workload (X [2048, 2048] BF16, gate/up [8192, 2048], down [2048, 8192]):

  fp8_observe(X)        observer update (max) on the batch
  gated_mlp_fp8(...)    quantize X once -> gate and up GEMMs with the
                        SwiGLU-FP8 epilogue (one kernel) -> down GEMM

Inputs are seeded synthetic draws (mlp_fp8_quant_amd.workloads), resident in
HBM before timing; weights are RTN-quantized and all static scales calibrated
on the GPU with the library's own observer and quantize calls.

Printed: one JSON line.  ``value`` is gated-MLP TFLOP/s (3 GEMMs, 2*M*N*K
each, over the step time).  ``roofline`` is for the dominant kernel (the
fused gate/up GEMMs with the SwiGLU-FP8 epilogue), with its average launch
time measured with HIP events on the stream it runs on.  ``cpu_baseline`` times the CPU oracle on a row
sample of the same workload (rank 0, N=1 only).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 gated-MLP TFLOP/s (+% of FP8 MFMA peak); quant/SwiGLU GB/s (% HBM)"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0      # MI355X dense F16/BF16 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E


def time_launches(torch, stream, f, reps, warm=2):
    """Average time in microseconds of `reps` back-to-back calls f(r), r the
    repetition index, after `warm` untimed calls: one pair of HIP events on
    `stream` around the timed calls, no host synchronization between them."""
    for r in range(warm):
        f(r)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        f(r)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="rows of X in the oracle's timed sample")
    p.add_argument("--no-large", action="store_true",
                   help="skip the large-MLP-size elementwise measurement")
    p.add_argument("--copy-calib-mb", type=int, default=0,
                   help="also run one plain device copy of this many MiB (a "
                        "known-size reference for the profiler's byte counters)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for {args.gpus}); "
              "the path has no multi-GPU code", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mlp_fp8_quant_amd as fp8
    from mlp_fp8_quant_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    wl = workloads.gen_tower_mlp()
    M, H = wl.x.shape
    I = wl.weights["gate"].shape[0]

    def dbf(b):
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

    x = dbf(wl.x)
    q, s = {}, {}
    for k, w in wl.weights.items():
        q[k], s[k] = fp8.rtn_weight(dbf(w))
    st_x = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st_x, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st_x)
    qx = fp8.fp8_quant_static(x, sx)
    G = fp8.fp8_linear(qx, q["gate"], sx, s["gate"])
    U = fp8.fp8_linear(qx, q["up"], sx, s["up"])
    st_h = fp8.new_observer_state(dev)
    fp8.fp8_observe_swiglu(G, U, st_h, fp8.OBS_MAX)
    sh = fp8.fp8_scale_from_state(st_h)
    y = torch.empty_like(x)
    ws = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8, device=dev)
    st_step = fp8.new_observer_state(dev)

    def step(accum):
        fp8.fp8_observe(x, st_step, fp8.OBS_MAX)
        fp8.gated_mlp_fp8(x, sx, q["gate"], s["gate"], q["up"], s["up"], sh,
                          q["down"], s["down"], out=y, workspace=ws, accum=accum)

    def timed_steps(accum):
        for _ in range(args.warmup):
            step(accum)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            step(accum)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    gemm_flops = 2.0 * M * I * H * 3
    ms_step = timed_steps(fp8.ACC_EXACT)
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    ms_step_fp8 = timed_steps(fp8.ACC_FP8_MFMA)

    # Per-kernel launch times: the composite's launch sequence issued as its
    # five parts (bitwise the same kernels), HIP events between them, on the
    # same stream.  Averaged over `steps` repetitions.
    qxb = ws[:M * H].view(M, H)
    Gb = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    Ub = torch.empty_like(Gb)
    qh = torch.empty((M, I), dtype=torch.uint8, device=dev)
    names = ["quant", "gate_up_swiglu", "down", "gate", "up", "silu"]

    def per_kernel(accum):
        # average launch time of each kernel of the step: `reps` launches of
        # that kernel back to back on the stream, bracketed by one pair of
        # HIP events on that stream (no host sync, no event between them)
        reps = max(args.steps, 10)
        calls = {
            "quant": lambda: fp8.fp8_quant_static(x, sx, out=qxb),
            "gate_up_swiglu": lambda: fp8.fp8_gate_up_swiglu(
                qxb, q["gate"], sx, s["gate"], q["up"], s["up"], sh, out=qh, accum=accum),
            "gate": lambda: fp8.fp8_linear(qxb, q["gate"], sx, s["gate"], out=Gb, accum=accum),
            "up": lambda: fp8.fp8_linear(qxb, q["up"], sx, s["up"], out=Ub, accum=accum),
            "silu": lambda: fp8.silu_mul_2in_fp8(Gb, Ub, sh, out=qh),
            "down": lambda: fp8.fp8_linear(qh, q["down"], sh, s["down"], out=y, accum=accum),
        }
        return {n: time_launches(torch, stream, lambda r, c=calls[n]: c(), reps, warm=3)
                for n in names}

    us = per_kernel(fp8.ACC_EXACT)
    us8 = per_kernel(fp8.ACC_FP8_MFMA)

    gate_flops = 2.0 * M * I * H
    fused_flops = 2 * gate_flops
    quant_bytes = 3.0 * M * H
    silu_bytes = 5.0 * M * I

    def tflops(fl, t_us):
        return fl / (t_us * 1e-6) / 1e12

    kernels = {
        "quant": {"us": us["quant"], "GB/s": quant_bytes / us["quant"] / 1e3,
                  "bytes": quant_bytes,
                  "note": "12 MB per launch: bound by launch and one memory round trip, not by "
                          "bandwidth; elementwise_large.quant_16384x5120 is the HBM-bound size"},
        "gate_up_swiglu": {"us": us["gate_up_swiglu"], "flops": fused_flops,
                           "TFLOP/s": tflops(fused_flops, us["gate_up_swiglu"])},
        "down": {"us": us["down"], "flops": gate_flops,
                 "TFLOP/s": tflops(gate_flops, us["down"])},
        "parts (not in the step)": {
            "gate_us": us["gate"], "gate_TFLOP/s": tflops(gate_flops, us["gate"]),
            "up_us": us["up"],
            "silu_us": us["silu"], "silu_GB/s": silu_bytes / us["silu"] / 1e3},
    }
    kernels["quant"]["frac_hbm"] = kernels["quant"]["GB/s"] / HBM_PEAK_GBS

    # dominant kernel of the step: the fused gate/up GEMMs with the SwiGLU-FP8
    # epilogue.  The default engine runs on the F16 matrix cores (FP8 codes
    # decoded exactly in the kernel): its peak is the dense F16 MFMA rate.
    fused = tflops(fused_flops, us["gate_up_swiglu"])
    roofline = {
        "kernel": f"gate/up GEMMs + SwiGLU-FP8 epilogue (exact engine, f16 MFMA) "
                  f"M={M} I={I} H={H}",
        "bound": "mfma", "achieved": fused, "peak": F16_PEAK_TFLOPS,
        "unit": "TFLOP/s", "frac": fused / F16_PEAK_TFLOPS,
        "traffic": recorded_traffic(f"gate_up_swiglu_exact_{M}x{I}x{H}"),
    }
    f8 = tflops(fused_flops, us8["gate_up_swiglu"])
    fp8_engine = {
        "value": gemm_flops / (ms_step_fp8 * 1e-3) / 1e12, "unit": "TFLOP/s",
        "ms_per_step": ms_step_fp8,
        "kernels_us": us8,
        "roofline": {"kernel": "gate/up GEMMs + SwiGLU-FP8 epilogue (FP8 MFMA engine)",
                     "bound": "mfma", "achieved": f8, "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": f8 / FP8_PEAK_TFLOPS},
    }

    large = None if args.no_large else elementwise_large(fp8, torch, dev, stream)
    rowwise = None if args.no_large else per_row_fp8(fp8, torch, dev, stream, M, H, I)
    topology = None if args.no_large else fused_topology(fp8, torch, dev, stream, qx, sx, sh, q, s)
    big_mlp = None if args.no_large else large_mlp(fp8, torch, dev, stream)
    towers = None if args.no_large else two_tower_layer(fp8, torch, dev, stream)

    if args.copy_calib_mb > 0:
        n = args.copy_calib_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows)

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "H": H, "I": I,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
        "fp8_mfma_engine": fp8_engine,
        "elementwise_large": large,
        "roofline_hbm": None if large is None else [
            {"kernel": k, "bound": "hbm", "achieved": large[k]["GB/s"], "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": large[k]["GB/s"] / HBM_PEAK_GBS,
             "bytes_per_launch": large[k]["bytes"], "traffic": None}
            for k in ("quant_16384x5120", "silu_16384x25600")],
        "per_row_fp8": rowwise,
        "fused_topology": topology,
        "large_mlp": big_mlp,
        "two_tower_layer": towers,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))


def fused_topology(fp8, torch, dev, stream, qx, sx, sh, q, s):
    """The topology the split path replaces, timed beside it (pull request
    "Load static FP8 Cosmos3 Nano/Super checkpoints without re-quantizing
    them": split GEMMs cost the same as fused ones, the fused group loses each
    member's own scale).  Gated MLP at the bench workload: the split path's
    fused gate/up + SwiGLU kernel; the fused topology (gate and up
    re-quantized onto max(s), one [M, 2I] GEMM, one-input SwiGLU); and the two
    split GEMMs written into column slices of one [M, 2I] buffer (row stride
    2I) + one-input SwiGLU.  Split Q/K/V [3072, 4096] x 3 * [4096, 4096]
    against one [3072, 12288] GEMM.  Also the share of codes the
    re-quantization changed (gate and up)."""
    def timed(f, reps=20):
        return time_launches(torch, stream, lambda r: f(), reps, warm=2)

    out = {}
    M, I = qx.shape[0], q["gate"].shape[0]
    group = torch.cat([s["gate"], s["up"]])
    rg = fp8.fp8_requantize_onto_max(q["gate"], s["gate"], group)
    ru = fp8.fp8_requantize_onto_max(q["up"], s["up"], group)
    smax = torch.max(group).reshape(1)
    wf = torch.cat([rg, ru])
    out["requantized_codes_changed"] = {
        "gate": float((rg != q["gate"]).float().mean()), "up": float((ru != q["up"]).float().mean()),
        "scale_ratio": float(torch.min(group) / torch.max(group))}
    qh = torch.empty((M, I), dtype=torch.uint8, device=dev)
    y2 = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    out["split_fused_kernel_us"] = timed(lambda: fp8.fp8_gate_up_swiglu(
        qx, q["gate"], sx, s["gate"], q["up"], s["up"], sh, out=qh))
    out["fused_topology_us"] = timed(lambda: (fp8.fp8_linear(qx, wf, sx, smax, out=y2),
                                              fp8.silu_mul_fp8(y2, sh, out=qh)))
    out["split_into_slices_us"] = timed(lambda: (
        fp8.fp8_linear_into(qx, q["gate"], sx, s["gate"], y2, col0=0),
        fp8.fp8_linear_into(qx, q["up"], sx, s["up"], y2, col0=I),
        fp8.silu_mul_fp8(y2, sh, out=qh)))
    del y2, rg, ru, wf
    # split vs fused Q/K/V at the split-QKV workload shape
    Mq, Hq = 3072, 4096
    qa = torch.randint(0, 0x7E, (Mq, Hq), dtype=torch.uint8, device=dev)
    ws = [torch.randint(0, 0x7E, (Hq, Hq), dtype=torch.uint8, device=dev) for _ in range(3)]
    sc = torch.tensor([1e-3], device=dev)
    ys = [torch.empty((Mq, Hq), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    wcat = torch.cat(ws)
    ycat = torch.empty((Mq, 3 * Hq), dtype=torch.bfloat16, device=dev)
    out["qkv_split_3_gemms_us"] = timed(lambda: [fp8.fp8_linear(qa, w, sc, sc, out=y) for w, y in zip(ws, ys)])
    out["qkv_fused_1_gemm_us"] = timed(lambda: fp8.fp8_linear(qa, wcat, sc, sc, out=ycat))
    # the split path as shipped: qkv_fp8 (quantize once + one grouped launch)
    xq = torch.randn((Mq, Hq), device=dev).to(torch.bfloat16)
    wsq = torch.empty(fp8.qkv_fp8_workspace(Mq, Hq), dtype=torch.uint8, device=dev)
    out["qkv_fp8_composite_us"] = timed(lambda: fp8.qkv_fp8(xq, sc, ws[0], sc, ws[1], sc, ws[2], sc,
                                                            outs=ys, workspace=wsq))
    out["qkv_quantize_us"] = timed(lambda: fp8.fp8_quant_static(xq, sc, out=wsq[:Mq * Hq].view(Mq, Hq)))
    del qa, ws, ys, wcat, ycat, xq, wsq
    torch.cuda.empty_cache()
    return out


def per_row_fp8(fp8, torch, dev, stream, M, H, I):
    """Per-row FP8 (per-token activation / per-channel weight scales) beside
    the per-tensor path: per-token quantization of the gen MLP's X [M, H] and of
    the large MLP's X [16384, 5120] (3 B per element), and the gate projection
    [M, I, H] with per-row scales on both engines (TFLOP/s)."""
    def timed(f, reps):
        return time_launches(torch, stream, f, reps, warm=2)

    out = {}
    for rows, k, reps in ((M, H, 50), (16384, 5120, 20)):
        xs = [torch.randn((rows, k), device=dev).to(torch.bfloat16) for _ in range(3)]
        q = torch.empty((rows, k), dtype=torch.uint8, device=dev)
        sc = torch.empty(rows, dtype=torch.float32, device=dev)
        us = timed(lambda r: fp8.fp8_quant_per_row(xs[r % 3], out=q, scales=sc), reps)
        out[f"quant_per_row_{rows}x{k}"] = {"us": us, "bytes": 3 * rows * k,
                                            "GB/s": 3 * rows * k / us / 1e3,
                                            "frac_hbm": 3 * rows * k / us / 1e3 / HBM_PEAK_GBS}
        del xs, q, sc
    x = torch.randn((M, H), device=dev).to(torch.bfloat16)
    w = (torch.randn((I, H), device=dev) * 0.02).to(torch.bfloat16)
    qx, sx = fp8.fp8_quant_per_row(x)
    qw, sw = fp8.fp8_quant_per_row(w)
    y = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    fl = 2.0 * M * I * H
    for eng, name in ((fp8.ACC_EXACT, "exact"), (fp8.ACC_FP8_MFMA, "fp8_mfma")):
        us = timed(lambda r: fp8.fp8_linear_rowwise(qx, qw, sx, sw, out=y, accum=eng), 20)
        out[f"linear_rowwise_{name}_{M}x{I}x{H}"] = {"us": us, "TFLOP/s": fl / us / 1e6}
    del x, w, qx, qw, y
    torch.cuda.empty_cache()
    return out


def large_mlp(fp8, torch, dev, stream):
    """The large compute-bound gated MLP (X [16384, 5120] N(0,1) with 0.5%
    x20 outliers; gate/up [25600, 5120] and down [5120, 25600] N(0, 0.015),
    RTN per tensor on the GPU; shared gate/up input scale amax(X)/448; down
    input scale amax(silu(G) * U)/448 from the library's own observer on this
    X): average time of the whole gated_mlp_fp8 call and of its two GEMM
    launches, both engines.  Inputs are drawn on the GPU (seeded) for speed."""
    M, H, I = 16384, 5120, 25600
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)

    def timed(f, reps=4):
        return time_launches(torch, stream, lambda r: f(), reps, warm=1)

    xf = torch.randn((M, H), device=dev, generator=gen)
    xf = torch.where(torch.rand((M, H), device=dev, generator=gen) < 0.005, xf * 20, xf)
    x = xf.to(torch.bfloat16)
    del xf
    q, s = {}, {}
    for k, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = (torch.randn(shape, device=dev, generator=gen) * 0.015).to(torch.bfloat16)
        q[k], s[k] = fp8.rtn_weight(w)
        del w
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st)
    qx = fp8.fp8_quant_static(x, sx)
    G = fp8.fp8_linear(qx, q["gate"], sx, s["gate"])
    U = fp8.fp8_linear(qx, q["up"], sx, s["up"])
    sth = fp8.new_observer_state(dev)
    fp8.fp8_observe_swiglu(G, U, sth, fp8.OBS_MAX)
    sh = fp8.fp8_scale_from_state(sth)
    del G, U
    torch.cuda.empty_cache()
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8, device=dev)
    qh = torch.empty((M, I), dtype=torch.uint8, device=dev)
    gemm_flops = 3 * 2.0 * M * I * H
    out = {"workload": f"large_mlp_M{M}_H{H}_I{I}", "gemm_flops": gemm_flops}
    for name, acc, peak in (("exact", fp8.ACC_EXACT, F16_PEAK_TFLOPS),
                            ("fp8_mfma", fp8.ACC_FP8_MFMA, FP8_PEAK_TFLOPS)):
        t = timed(lambda: fp8.gated_mlp_fp8(x, sx, q["gate"], s["gate"], q["up"], s["up"], sh,
                                            q["down"], s["down"], out=y, workspace=ws, accum=acc))
        tf = timed(lambda: fp8.fp8_gate_up_swiglu(qx, q["gate"], sx, s["gate"], q["up"], s["up"],
                                                  sh, out=qh, accum=acc))
        td = timed(lambda: fp8.fp8_linear(qh, q["down"], sh, s["down"], out=y, accum=acc))
        f_fused = 2 * 2.0 * M * I * H / (tf * 1e-6) / 1e12
        f_down = 2.0 * M * I * H / (td * 1e-6) / 1e12
        out[name] = {
            "gated_mlp_us": t, "TFLOP/s": gemm_flops / (t * 1e-6) / 1e12,
            "gate_up_swiglu_us": tf, "gate_up_swiglu_TFLOP/s": f_fused,
            "gate_up_swiglu_frac_peak": f_fused / peak,
            "down_us": td, "down_TFLOP/s": f_down, "down_frac_peak": f_down / peak,
            "peak_TFLOP/s": peak,
        }
    del x, qx, qh, y, ws, q
    torch.cuda.empty_cache()
    return out


def two_tower_layer(fp8, torch, dev, stream):
    """One decoder layer's FP8 Linear set for both towers (H=4096, I=12288;
    und M=512 tokens, gen M=4096): per tower qkv_fp8 (one quantization, three
    GEMMs), the o projection (its own quantize + GEMM) and gated_mlp_fp8.
    Weights N(0, 0.02) RTN per tensor on the GPU; the layer's activations are
    drawn N(0, 1) with 0.5% x20 outliers (attention itself is not on this
    path, so the o-projection input is drawn too); input scales are each
    site's amax/448 from the library's max observer on that input, down's
    from fp8_observe_swiglu.  Average time of the whole set, both engines."""
    H, I = 4096, 12288
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)

    def act(M):
        xf = torch.randn((M, H), device=dev, generator=gen)
        xf = torch.where(torch.rand((M, H), device=dev, generator=gen) < 0.005, xf * 20, xf)
        return xf.to(torch.bfloat16)

    def weight(n, k):
        return fp8.rtn_weight((torch.randn((n, k), device=dev, generator=gen) * 0.02)
                              .to(torch.bfloat16))

    def scale_of(x):
        st = fp8.new_observer_state(dev)
        fp8.fp8_observe(x, st, fp8.OBS_MAX)
        return fp8.fp8_scale_from_state(st)

    towers = {}
    for name, M in (("und", 512), ("gen", 4096)):
        t = {"M": M, "x_qkv": act(M), "x_o": act(M), "x_mlp": act(M)}
        for k, (n, kk) in {"q": (H, H), "k": (H, H), "v": (H, H), "o": (H, H),
                           "gate": (I, H), "up": (I, H), "down": (H, I)}.items():
            t["w_" + k], t["s_" + k] = weight(n, kk)
        t["sx_qkv"], t["sx_o"], t["sx_mlp"] = (scale_of(t["x_qkv"]), scale_of(t["x_o"]),
                                              scale_of(t["x_mlp"]))
        qx = fp8.fp8_quant_static(t["x_mlp"], t["sx_mlp"])
        G = fp8.fp8_linear(qx, t["w_gate"], t["sx_mlp"], t["s_gate"])
        U = fp8.fp8_linear(qx, t["w_up"], t["sx_mlp"], t["s_up"])
        sth = fp8.new_observer_state(dev)
        fp8.fp8_observe_swiglu(G, U, sth, fp8.OBS_MAX)
        t["sh"] = fp8.fp8_scale_from_state(sth)
        del qx, G, U
        t["outs"] = tuple(torch.empty((M, H), dtype=torch.bfloat16, device=dev) for _ in range(3))
        t["ws_qkv"] = torch.empty(fp8.qkv_fp8_workspace(M, H), dtype=torch.uint8, device=dev)
        t["qo"] = torch.empty((M, H), dtype=torch.uint8, device=dev)
        t["yo"] = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        t["ws_mlp"] = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8,
                                  device=dev)
        t["y"] = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        t["flops"] = 2.0 * M * H * H * 4 + 3 * 2.0 * M * I * H
        towers[name] = t

    def layer(t, acc):
        fp8.qkv_fp8(t["x_qkv"], t["sx_qkv"], t["w_q"], t["s_q"], t["w_k"], t["s_k"],
                    t["w_v"], t["s_v"], outs=t["outs"], workspace=t["ws_qkv"], accum=acc)
        fp8.fp8_quant_static(t["x_o"], t["sx_o"], out=t["qo"])
        fp8.fp8_linear(t["qo"], t["w_o"], t["sx_o"], t["s_o"], out=t["yo"], accum=acc)
        fp8.gated_mlp_fp8(t["x_mlp"], t["sx_mlp"], t["w_gate"], t["s_gate"], t["w_up"],
                          t["s_up"], t["sh"], t["w_down"], t["s_down"], out=t["y"],
                          workspace=t["ws_mlp"], accum=acc)

    def timed(f, reps=20):
        return time_launches(torch, stream, lambda r: f(), reps, warm=5)

    out = {"workload": "two_tower_layer_H4096_I12288_und512_gen4096",
           "gemm_flops": {k: t["flops"] for k, t in towers.items()}}
    for en, acc, peak in (("exact", fp8.ACC_EXACT, F16_PEAK_TFLOPS),
                          ("fp8_mfma", fp8.ACC_FP8_MFMA, FP8_PEAK_TFLOPS)):
        r = {}
        for k, t in towers.items():
            us = timed(lambda: layer(t, acc))
            r[k] = {"us": us, "TFLOP/s": t["flops"] / (us * 1e-6) / 1e12}
        us = timed(lambda: [layer(t, acc) for t in towers.values()])
        tot = sum(t["flops"] for t in towers.values())
        r["both_towers"] = {"us": us, "TFLOP/s": tot / (us * 1e-6) / 1e12,
                            "frac_peak": tot / (us * 1e-6) / 1e12 / peak}
        out[en] = r
    del towers
    torch.cuda.empty_cache()
    return out


def elementwise_large(fp8, torch, dev, stream):
    """The HBM-bound kernels at the large gated-MLP sizes (X [16384, 5120],
    G/U [16384, 25600], or G|U adjacent in one [16384, 51200] tensor for the
    one-input SwiGLU), where the working sets exceed the 256 MB MALL:
    average launch time over back-to-back launches (three rotating X copies
    for quantize), algorithmic GB/s, and the fraction of the 8 TB/s peak.
    A plain device copy of the SwiGLU's byte count is timed beside them."""
    def timed(f, reps):
        return time_launches(torch, stream, f, reps, warm=2)

    out = {}
    n = 16384 * 5120
    xs = [torch.randn(n, device=dev).to(torch.bfloat16) for _ in range(3)]
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    s = torch.tensor([0.02], device=dev)
    us = timed(lambda r: fp8.fp8_quant_static(xs[r % 3], s, out=q), 20)
    out["quant_16384x5120"] = {"us": us, "bytes": 3 * n, "GB/s": 3 * n / us / 1e3,
                               "frac_hbm": 3 * n / us / 1e3 / HBM_PEAK_GBS}
    del xs, q
    n = 16384 * 25600
    g = torch.randn(n, device=dev).to(torch.bfloat16)
    u = torch.randn(n, device=dev).to(torch.bfloat16)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    us = timed(lambda r: fp8.silu_mul_2in_fp8(g, u, s, out=q), 8)
    out["silu_16384x25600"] = {"us": us, "bytes": 5 * n, "GB/s": 5 * n / us / 1e3,
                               "frac_hbm": 5 * n / us / 1e3 / HBM_PEAK_GBS}
    # the swiglu_alpha / swiglu_beta variant (swigluoai shape) on the same data
    us = timed(lambda r: fp8.silu_mul_2in_fp8(g, u, s, out=q, alpha=1.702, beta=1.0), 8)
    out["silu_ab_16384x25600"] = {"us": us, "bytes": 5 * n, "GB/s": 5 * n / us / 1e3,
                                  "frac_hbm": 5 * n / us / 1e3 / HBM_PEAK_GBS}
    del q
    a = g.view(torch.uint8)
    b = torch.empty_like(a)
    us = timed(lambda r: b.copy_(a), 8)
    out["device_copy_same_bytes"] = {"us": us, "GB/s": 2 * a.numel() / us / 1e3}
    del g, u, a, b
    torch.cuda.empty_cache()
    # one-input SwiGLU: gate and up adjacent in one [16384, 2 x 25600] tensor
    x = torch.randn((16384, 2 * 25600), device=dev).to(torch.bfloat16)
    q = torch.empty((16384, 25600), dtype=torch.uint8, device=dev)
    us = timed(lambda r: fp8.silu_mul_fp8(x, s, out=q), 8)
    out["silu_1in_16384x25600"] = {"us": us, "bytes": 5 * n, "GB/s": 5 * n / us / 1e3,
                                   "frac_hbm": 5 * n / us / 1e3 / HBM_PEAK_GBS}
    del x, q
    torch.cuda.empty_cache()
    return out


def recorded_traffic(key):
    """HBM-side bytes per launch of a kernel, as recorded from rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by a plain copy of known size) in
    profiles/gemm_traffic.md, or None when that record is missing or was
    taken from a different version of the GEMM source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_traffic.md")
    src = os.path.join(ROOT, "mlp_fp8_quant_amd", "csrc", "gemm.hip")
    try:
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        for line in open(path):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 5 and cells[0] == key and cells[4] == digest:
                return {"fetch_bytes": float(cells[1]), "write_bytes": float(cells[2]),
                        "total_bytes": float(cells[1]) + float(cells[2]),
                        "algorithmic_bytes": float(cells[3])}
    except (OSError, ValueError):
        pass
    return None


def cpu_baseline(wl, rows):
    """The oracle, as it stands, on a row sample of the same workload: the
    whole chain (quantize X, exact gate/up GEMMs with the BF16 epilogue,
    FP8 SwiGLU, exact down GEMM) for the first `rows` rows of X.  Reported
    in the metric's unit: gated-MLP GEMM TFLOP/s of that sample."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import linear as olin
    from oracle.swiglu import silu_mul_f64, silu_mul_fp8

    x = wl.x[:rows]
    q, s = {}, {}
    for k, w in wl.weights.items():
        q[k], s[k] = olin.rtn_weight(w)
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    t = time.perf_counter()
    qx = olin.quant_static(x, sx)
    Sg, _ = olin.gemm_exact(qx, q["gate"])
    Su, _ = olin.gemm_exact(qx, q["up"])
    G = olin.epilogue_bf16(Sg, sx, s["gate"])
    U = olin.epilogue_bf16(Su, sx, s["up"])
    sh = olin.scale_from_amax(np.float32(np.max(np.abs(silu_mul_f64(G, U)))))
    qh = silu_mul_fp8(G, U, sh).reshape(G.shape)
    Sd, _ = olin.gemm_exact(qh, q["down"])
    olin.epilogue_bf16(Sd, sh, s["down"])
    dt = time.perf_counter() - t
    H = x.shape[1]
    I = q["gate"].shape[0]
    flops = 2.0 * rows * I * H * 3
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": dt,
            "sample": f"rows 0..{rows - 1} of X through the whole gated MLP "
                      f"(M={rows}, H={H}, I={I}); float64 exact GEMMs"}


if __name__ == "__main__":
    main()
