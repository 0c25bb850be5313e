"""Benchmark of the static FP8 gated-MLP hot path on one MI355X.

One step = one pass of the whole path over one batch of the large
compute-bound gated MLP, the largest workload that fits one GPU (X
[16384, 5120] BF16 with 0.5% x20 outliers; gate/up [25600, 5120] and down
[5120, 25600], N(0, 0.015), RTN per tensor):

  fp8_observe(X)        observer update (max) on the batch
  gated_mlp_fp8(...)    quantize X once -> gate and up GEMMs with the
                        SwiGLU-FP8 epilogue (one kernel) -> down GEMM

on the exact engine (FP8 codes decoded exactly in the kernel and multiplied
on the F16 matrix cores with FP32 accumulation; the engine that meets the
GEMM tolerance).  Inputs are seeded synthetic draws
(mlp_fp8_quant_amd.workloads), resident in HBM before timing; weights are
RTN-quantized and all static scales calibrated on the GPU with the library's
own observer and quantize calls.

Printed: one JSON line.  ``value`` is gated-MLP TFLOP/s (3 GEMMs, 2*M*N*K
each, over the step time).  ``roofline`` is for the dominant kernel (the
fused gate/up GEMMs with the SwiGLU-FP8 epilogue) against the FP8 dense MFMA
peak the metric names, with its average launch time measured with HIP events
on the stream it runs on, and beside the rate the matrix cores sustain on the
step's own operand codes with nothing else in the loop (``mfma_ceiling``).
``cpu_baseline`` times the CPU oracle on a bounded
block of the same workload.  Further blocks: the native FP8 MFMA engine
(flagged: below the path's tolerance), vendor-library GEMMs at the same
shape, the gen-tower gated MLP, the HBM-bound kernels beside a read/write
ceiling of their byte mix, per-row FP8, the fused-topology comparison and
the two-tower layer under both calibrated scale sets.
"""

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 gated-MLP TFLOP/s (+% of FP8 MFMA peak); quant/SwiGLU GB/s (% HBM)"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0      # MI355X dense F16/BF16 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
FP8_ENGINE_NOTE = ("native FP8 MFMA: each 8-product group is summed on a grid 13 bits below "
                   "its largest product, which misses the path's GEMM tolerance "
                   "(1e-5 sum|terms|) on part of the outputs; reported for context only")


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


def launch_stats(torch, stream, f, reps, warm=2):
    """Median and minimum per-launch time in microseconds of `reps`
    back-to-back calls f(r): an event recorded on `stream` between
    consecutive calls, no host synchronization between them."""
    for r in range(warm):
        f(r)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        f(r)
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    return {"us_median": d[reps // 2], "us_min": d[0], "launches": reps}


def mfma_ceiling_against(fp8, torch, stream, kernel, flops, a, b, accum, rounds=3,
                         window_s=0.3, clock=None):
    """A GEMM kernel beside the MFMA ceiling on the same operand codes: the
    library's dense MFMA loop (fp8mot_mfma_ceiling; fragments taken from the
    codes in a and b, nothing else in the loop) sized to last about as long
    as one kernel launch, the two timed alternately `rounds` times in
    windows of ~window_s each (so both run in the same power and clock
    state); medians.  kernel(r) launches the GEMM, which does `flops`.  With a
    ClockSampler, the GFX clock is also sampled over ~1.5 s of sustained
    ceiling launches."""
    sink = torch.zeros(1, dtype=torch.float32, device=a.device)
    probe_iters = 1000
    t_probe = time_launches(torch, stream,
                            lambda r: fp8.mfma_ceiling(a, b, probe_iters, sink, accum), 3, warm=1)
    t_kernel = time_launches(torch, stream, kernel, 2, warm=1)
    iters = max(probe_iters, int(probe_iters * t_kernel / t_probe))
    per_launch = fp8.mfma_ceiling(a, b, iters, sink, accum)
    reps = max(3, int(window_s * 1e6 / t_kernel))
    ks, cs = [], []
    for _ in range(rounds):
        ks.append(time_launches(torch, stream, kernel, reps, warm=1))
        cs.append(time_launches(torch, stream,
                                lambda r: fp8.mfma_ceiling(a, b, iters, sink, accum), reps, warm=1))
    k, c = sorted(ks)[rounds // 2], sorted(cs)[rounds // 2]
    sclk = None
    if clock is not None:
        sclk = sustained_clock(lambda: fp8.mfma_ceiling(a, b, iters, sink, accum), clock, torch)
    torch.cuda.synchronize()
    assert float(sink.item()) == 0.0
    ceiling = per_launch / c / 1e6
    achieved = flops / k / 1e6
    return {"ceiling_TFLOP/s": ceiling, "ceiling_launch_us": c, "ceiling_iters": iters,
            "kernel_TFLOP/s_same_windows": achieved, "kernel_launch_us_same_windows": k,
            "frac_of_ceiling": achieved / ceiling, "sclk_during_ceiling": sclk}


def sustained_clock(fn, clock, torch, seconds=1.5, batch=10):
    """The GFX clock while fn() runs back to back for ~seconds: batches of
    launches with the next batch queued before waiting on the previous one,
    so the GPU never idles while `clock` samples; sampling stops while the
    last batch is still queued."""
    clock.start()
    prev = None
    t_end = time.perf_counter() + seconds
    while True:
        for _ in range(batch):
            fn()
        ev = torch.cuda.Event()
        ev.record()
        if prev is not None:
            prev.synchronize()
        prev = ev
        if time.perf_counter() >= t_end:
            break
    sclk = clock.stop()
    torch.cuda.synchronize()
    return sclk


class ClockSampler:
    """Samples the GPU's graphics clock on a host thread while GPU work runs:
    amdsmi's current GFX clock of each XCD from the firmware's metrics table
    (mean over the XCDs per sample).  The table refreshes every ~100-300 ms,
    so only a sustained run of a second or more gives a meaningful figure;
    the first `skip_s` seconds of samples are dropped."""

    def __init__(self, period_s=0.02):
        self.period = period_s
        self.samples = []
        self.err = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception as e:   # no management interface: report null
            self._smi = None
            self.err = f"{type(e).__name__}: {e}"

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        xs = [float(v) for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float))]
        if not xs and isinstance(m.get("current_gfxclk"), (int, float)):
            xs = [float(m["current_gfxclk"])]
        return sum(xs) / len(xs) if xs else None

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append((time.perf_counter() - t0, v))
            except Exception as e:
                self.err = f"{type(e).__name__}: {e}"
                return
            time.sleep(self.period)

    def start(self):
        self.samples = []
        self._stop.clear()
        if self._smi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self, skip_s=0.3):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        vals = sorted(v for t, v in self.samples if t >= skip_s)
        if not vals:
            return {"mhz_median": None, "samples": 0, "error": self.err}
        return {"mhz_median": vals[len(vals) // 2], "mhz_min": vals[0], "mhz_max": vals[-1],
                "samples": len(vals),
                "source": "amdsmi gpu metrics current_gfxclks, mean over XCDs per sample"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=16384,
                   help="rows of X in the oracle's timed block")
    p.add_argument("--cpu-channels", type=int, default=5120,
                   help="intermediate channels in the oracle's timed block")
    p.add_argument("--no-blocks", action="store_true",
                   help="only the headline step and its kernels (for profiling runs)")
    p.add_argument("--blocks", default="gen_mlp,elementwise_large,per_row_fp8,fused_topology,"
                                       "two_tower_layer,library_references,single_linear",
                   help="comma-separated extra blocks to run")
    p.add_argument("--copy-calib-mb", type=int, default=0,
                   help="also run one plain device copy of this many MiB (a "
                        "known-size reference for the profiler's byte counters)")
    return p.parse_args()


def dev_bf16(torch, bits, dev):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def tflops(fl, t_us):
    return fl / (t_us * 1e-6) / 1e12


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for {args.gpus}); "
              "the path has no multi-GPU code", file=sys.stderr)
        sys.exit(2)

    import torch

    import mlp_fp8_quant_amd as fp8
    from mlp_fp8_quant_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    clock = ClockSampler()

    # ---- the large gated MLP (headline workload) ----
    wl = workloads.super_mlp()
    M, H = wl.x.shape
    I = wl.weights["gate"].shape[0]
    x = dev_bf16(torch, wl.x, dev)
    q, s = {}, {}
    for k, w in wl.weights.items():
        q[k], s[k] = fp8.rtn_weight(dev_bf16(torch, w, dev))
    wl_cpu = wl
    st_x = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st_x, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st_x)
    qx = fp8.fp8_quant_static(x, sx)
    G = fp8.fp8_linear(qx, q["gate"], sx, s["gate"])
    U = fp8.fp8_linear(qx, q["up"], sx, s["up"])
    st_h = fp8.new_observer_state(dev)
    fp8.fp8_observe_swiglu(G, U, st_h, fp8.OBS_MAX)
    sh = fp8.fp8_scale_from_state(st_h)
    del G, U
    torch.cuda.empty_cache()
    y = torch.empty_like(x)
    ws = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8, device=dev)
    st_step = fp8.new_observer_state(dev)

    def step(accum):
        fp8.fp8_observe(x, st_step, fp8.OBS_MAX)
        fp8.gated_mlp_fp8(x, sx, q["gate"], s["gate"], q["up"], s["up"], sh,
                          q["down"], s["down"], out=y, workspace=ws, accum=accum)

    def timed_steps(accum, steps, warmup):
        for _ in range(warmup):
            step(accum)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            step(accum)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    gemm_flops = 2.0 * M * I * H * 3
    fused_flops = 2 * 2.0 * M * I * H
    down_flops = 2.0 * M * I * H
    ms_step = timed_steps(fp8.ACC_EXACT, args.steps, args.warmup)
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    # the clock under this load: the same step, sustained for ~1.5 s
    sclk_step = sustained_clock(lambda: step(fp8.ACC_EXACT), clock, torch)

    # kernels of the step, each timed alone: back-to-back launches on the
    # stream they run on, one pair of HIP events around them
    qxb = ws[:M * H].view(M, H)
    qh = ws[fp8.gated_mlp_fp8_workspace(M, H, 0):][:M * I].view(M, I)

    def kernel_times(accum, reps):
        calls = {
            "observe": lambda r: fp8.fp8_observe(x, st_step, fp8.OBS_MAX),
            "quant": lambda r: fp8.fp8_quant_static(x, sx, out=qxb),
            "gate_up_swiglu": lambda r: fp8.fp8_gate_up_swiglu(
                qxb, q["gate"], sx, s["gate"], q["up"], s["up"], sh, out=qh, accum=accum),
            "down": lambda r: fp8.fp8_linear(qh, q["down"], sh, s["down"], out=y, accum=accum),
        }
        out, dist = {}, {}
        for n, f in calls.items():
            reps_n = reps if n in ("gate_up_swiglu", "down") else 4 * reps
            out[n] = time_launches(torch, stream, f, reps_n, warm=2)
            dist[n] = launch_stats(torch, stream, f, reps_n, warm=0)
        return out, dist

    us, us_dist = kernel_times(fp8.ACC_EXACT, 10)
    kernels = {
        "observe": {"us": us["observe"], "bytes": 2.0 * M * H,
                    "GB/s": 2.0 * M * H / us["observe"] / 1e3},
        "quant": {"us": us["quant"], "bytes": 3.0 * M * H,
                  "GB/s": 3.0 * M * H / us["quant"] / 1e3,
                  "frac_hbm": 3.0 * M * H / us["quant"] / 1e3 / HBM_PEAK_GBS},
        "gate_up_swiglu": {"us": us["gate_up_swiglu"], "flops": fused_flops,
                           "TFLOP/s": tflops(fused_flops, us["gate_up_swiglu"]),
                           "frac_fp8_peak": tflops(fused_flops, us["gate_up_swiglu"]) / FP8_PEAK_TFLOPS},
        "down": {"us": us["down"], "flops": down_flops,
                 "TFLOP/s": tflops(down_flops, us["down"]),
                 "frac_fp8_peak": tflops(down_flops, us["down"]) / FP8_PEAK_TFLOPS},
    }
    for n, d in us_dist.items():   # per-launch spread beside the back-to-back average
        kernels[n].update(d)
    fused = tflops(fused_flops, us["gate_up_swiglu"])
    roofline = {
        "kernel": f"gate/up GEMMs + SwiGLU-FP8 epilogue, exact engine (F16 MFMA on exactly "
                  f"decoded FP8 codes), M={M} I={I} H={H}",
        "bound": "mfma", "achieved": fused, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": fused / FP8_PEAK_TFLOPS,
        "traffic": recorded_traffic(f"gate_up_swiglu_exact_{M}x{I}x{H}", "gemm.hip"),
        "launch_us": us["gate_up_swiglu"], "flops_per_launch": fused_flops,
        "frac_f16_peak": fused / F16_PEAK_TFLOPS,
    }
    # the same kernel beside what the F16 matrix cores sustain on the step's own
    # operand codes with nothing else in the loop
    fused_call = lambda r: fp8.fp8_gate_up_swiglu(qxb, q["gate"], sx, s["gate"], q["up"], s["up"],
                                                  sh, out=qh, accum=fp8.ACC_EXACT)
    roofline["mfma_ceiling"] = {
        "kind": "dense v_mfma_f32_32x32x16_f16 loop on fragments of the step's own X and W_gate "
                "codes (fp8mot_mfma_ceiling), timed alternately with the kernel",
        **mfma_ceiling_against(fp8, torch, stream, fused_call, fused_flops, qxb, q["gate"],
                               fp8.ACC_EXACT, clock=clock)}

    # the native FP8 MFMA engine, same workload (context only)
    ms8 = timed_steps(fp8.ACC_FP8_MFMA, max(args.steps // 2, 5), 3)
    us8, _ = kernel_times(fp8.ACC_FP8_MFMA, 5)
    f8 = tflops(fused_flops, us8["gate_up_swiglu"])
    fp8_engine = {
        "meets_tolerance": False, "note": FP8_ENGINE_NOTE,
        "value": gemm_flops / (ms8 * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms8,
        "kernels_us": us8,
        "gate_up_swiglu_frac_fp8_peak": f8 / FP8_PEAK_TFLOPS,
        "down_frac_fp8_peak": tflops(down_flops, us8["down"]) / FP8_PEAK_TFLOPS,
    }
    fused8_call = lambda r: fp8.fp8_gate_up_swiglu(qxb, q["gate"], sx, s["gate"], q["up"], s["up"],
                                                   sh, out=qh, accum=fp8.ACC_FP8_MFMA)
    fp8_engine["mfma_ceiling"] = {
        "kind": "dense native FP8 v_mfma_scale_f32_32x32x64_f8f6f4 loop on fragments of the "
                "same codes, timed alternately with the FP8-engine fused kernel",
        **mfma_ceiling_against(fp8, torch, stream, fused8_call, fused_flops, qxb, q["gate"],
                               fp8.ACC_FP8_MFMA)}
    want = set() if args.no_blocks else set(args.blocks.split(","))
    refs = (library_references(fp8, torch, dev, stream, qxb, q, sx, s)
            if "library_references" in want else None)

    del x, q, qx, y, ws
    torch.cuda.empty_cache()

    blocks = {}
    if "gen_mlp" in want:
        blocks["gen_mlp"] = gen_mlp(fp8, torch, dev, stream, workloads)
    if "elementwise_large" in want:
        blocks["elementwise_large"] = elementwise_large(fp8, torch, dev, stream)
    if "per_row_fp8" in want:
        blocks["per_row_fp8"] = per_row_fp8(fp8, torch, dev, stream)
    if "fused_topology" in want:
        blocks["fused_topology"] = fused_topology(fp8, torch, dev, stream, workloads)
    if "two_tower_layer" in want:
        blocks["two_tower_layer"] = two_tower_layer(fp8, torch, dev, stream)
    if "single_linear" in want:
        blocks["single_linear"] = single_linear(fp8, torch, dev, stream, workloads)

    if args.copy_calib_mb > 0:
        n = args.copy_calib_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl_cpu, args.cpu_rows, args.cpu_channels)

    large = blocks.get("elementwise_large")
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 operands, f16 MFMA products, f32 accumulate",
        "data": "synthetic (seeded; mlp_fp8_quant_amd.workloads)",
        "config": {"workload": wl_cpu.name, "M": M, "H": H, "I": I, "engine": "exact",
                   "step": "fp8_observe(X) + gated_mlp_fp8", "parallelism": "none (1 GPU)"},
        "frac_fp8_peak": value / FP8_PEAK_TFLOPS,
        "roofline": roofline, "cpu_baseline": cpu, "sclk_during_steps": sclk_step,
        "kernels": kernels, "fp8_mfma_engine": fp8_engine,
        "library_references": refs,
        "roofline_hbm": None if large is None else [
            {"kernel": k, "bound": "hbm", "achieved": large[k]["GB/s"], "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": large[k]["GB/s"] / HBM_PEAK_GBS,
             "bytes_per_launch": large[k]["bytes"],
             "ceiling_same_mix_GB/s": large[k]["ceiling_GB/s"],
             "frac_of_ceiling": large[k]["GB/s"] / large[k]["ceiling_GB/s"],
             "traffic": recorded_traffic(key, "elementwise.hip")}
            for k, key in (("quant_16384x5120", "quant_static_16384x5120"),
                           ("silu_16384x25600", "silu_mul_16384x25600"))],
        **blocks,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))


def library_references(fp8, torch, dev, stream, qx, q, sx, s):
    """Vendor-library GEMMs at the gate projection's shape (16384 x 25600 x
    5120) on the same operand values, for context (not this path): hipBLASLt
    F16 (torch.mm on the exactly decoded codes, FP32 accumulate) and hipBLASLt
    FP8 (torch._scaled_mm on the codes, whose FP8 MFMAs accumulate like this
    library's FP8 engine)."""
    out = {}
    M, H = qx.shape
    N = q["gate"].shape[0]
    fl = 2.0 * M * N * H

    def timed(f, reps=5):
        return time_launches(torch, stream, lambda r: f(), reps, warm=2)

    try:
        a16 = qx.view(torch.float8_e4m3fn).to(torch.float16)
        b16t = q["gate"].view(torch.float8_e4m3fn).to(torch.float16).t().contiguous()
        c16 = torch.empty((M, N), dtype=torch.float16, device=dev)
        t = timed(lambda: torch.mm(a16, b16t, out=c16))
        out["hipblaslt_f16"] = {"us": t, "TFLOP/s": tflops(fl, t),
                                "frac_f16_peak": tflops(fl, t) / F16_PEAK_TFLOPS}
        del a16, b16t, c16
    except Exception as e:   # report, do not fail the bench
        out["hipblaslt_f16"] = {"error": f"{type(e).__name__}: {e}"}
    try:
        a8 = qx.view(torch.float8_e4m3fn)
        b8 = q["gate"].view(torch.float8_e4m3fn)
        t = timed(lambda: torch._scaled_mm(a8, b8.t(), scale_a=sx, scale_b=s["gate"],
                                           out_dtype=torch.bfloat16))
        out["hipblaslt_fp8"] = {"us": t, "TFLOP/s": tflops(fl, t),
                                "frac_fp8_peak": tflops(fl, t) / FP8_PEAK_TFLOPS,
                                "meets_tolerance": False, "note": FP8_ENGINE_NOTE}
    except Exception as e:
        out["hipblaslt_fp8"] = {"error": f"{type(e).__name__}: {e}"}
    out["shape"] = f"{M}x{N}x{H}"
    torch.cuda.empty_cache()
    return out


def gen_mlp(fp8, torch, dev, stream, workloads):
    """The gen-tower gated MLP (X [2048, 2048], gate/up [8192, 2048], down
    [2048, 8192]): the same step at that size, and each kernel timed alone,
    both engines."""
    wl = workloads.gen_tower_mlp()
    M, H = wl.x.shape
    I = wl.weights["gate"].shape[0]
    x = dev_bf16(torch, wl.x, dev)
    q, s = {}, {}
    for k, w in wl.weights.items():
        q[k], s[k] = fp8.rtn_weight(dev_bf16(torch, w, dev))
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st)
    qx = fp8.fp8_quant_static(x, sx)
    G = fp8.fp8_linear(qx, q["gate"], sx, s["gate"])
    U = fp8.fp8_linear(qx, q["up"], sx, s["up"])
    sth = fp8.new_observer_state(dev)
    fp8.fp8_observe_swiglu(G, U, sth, fp8.OBS_MAX)
    sh = fp8.fp8_scale_from_state(sth)
    y = torch.empty_like(x)
    ws = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8, device=dev)
    qh = torch.empty((M, I), dtype=torch.uint8, device=dev)
    st_step = fp8.new_observer_state(dev)
    fl = 2.0 * M * I * H
    out = {"workload": wl.name}
    for name, acc in (("exact", fp8.ACC_EXACT), ("fp8_mfma", fp8.ACC_FP8_MFMA)):
        def stepf(r):
            fp8.fp8_observe(x, st_step, fp8.OBS_MAX)
            fp8.gated_mlp_fp8(x, sx, q["gate"], s["gate"], q["up"], s["up"], sh,
                              q["down"], s["down"], out=y, workspace=ws, accum=acc)
        t = time_launches(torch, stream, stepf, 100, warm=50)
        k = {
            "quant": time_launches(torch, stream, lambda r: fp8.fp8_quant_static(x, sx, out=qx), 100),
            "gate_up_swiglu": time_launches(torch, stream, lambda r: fp8.fp8_gate_up_swiglu(
                qx, q["gate"], sx, s["gate"], q["up"], s["up"], sh, out=qh, accum=acc), 50),
            "down": time_launches(torch, stream, lambda r: fp8.fp8_linear(
                qh, q["down"], sh, s["down"], out=y, accum=acc), 50),
            "gate_alone": time_launches(torch, stream, lambda r: fp8.fp8_linear(
                qx, q["gate"], sx, s["gate"], out=G, accum=acc), 50),
            "silu_alone": time_launches(torch, stream, lambda r: fp8.silu_mul_2in_fp8(
                G, U, sh, out=qh), 50),
        }
        out[name] = {"step_us": t, "TFLOP/s": 3 * fl / (t * 1e-6) / 1e12,
                     "kernels_us": k,
                     "gate_up_swiglu_TFLOP/s": tflops(2 * fl, k["gate_up_swiglu"]),
                     "down_TFLOP/s": tflops(fl, k["down"])}
        if acc == fp8.ACC_FP8_MFMA:
            out[name].update(meets_tolerance=False, note=FP8_ENGINE_NOTE)
    del x, q, qx, G, U, y, ws, qh
    torch.cuda.empty_cache()
    return out


def fused_topology(fp8, torch, dev, stream, workloads):
    """The topology the split path replaces, timed beside it (pull request
    "Load static FP8 Cosmos3 Nano/Super checkpoints without re-quantizing
    them": split GEMMs cost the same as fused ones, the fused group loses each
    member's own scale).  Gated MLP at the gen-tower size: the split path's
    fused gate/up + SwiGLU kernel; the fused topology (gate and up
    re-quantized onto max(s), one [M, 2I] GEMM, one-input SwiGLU); and the two
    split GEMMs written into column slices of one [M, 2I] buffer (row stride
    2I) + one-input SwiGLU.  Split Q/K/V [3072, 4096] x 3 * [4096, 4096]
    against one [3072, 12288] GEMM, and what a downstream per-row consumer of
    q and k (an RMS norm) costs on the split path's contiguous outputs and on
    the fused GEMM's column slices (row stride 3 * 4096).  Also the share of
    codes the re-quantization changed (gate and up)."""
    def timed(f, reps=20):
        return time_launches(torch, stream, lambda r: f(), reps, warm=2)

    wl = workloads.gen_tower_mlp()
    x = dev_bf16(torch, wl.x, dev)
    q, s = {}, {}
    for k in ("gate", "up"):
        q[k], s[k] = fp8.rtn_weight(dev_bf16(torch, wl.weights[k], dev))
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st)
    qx = fp8.fp8_quant_static(x, sx)
    sh = torch.tensor([0.01], dtype=torch.float32, device=dev)
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
    del y2, rg, ru, wf, x
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
    out["qkv_fp8_composite_TFLOP/s"] = tflops(3 * 2.0 * Mq * Hq * Hq, out["qkv_fp8_composite_us"])
    out["qkv_quantize_us"] = timed(lambda: fp8.fp8_quant_static(xq, sc, out=wsq[:Mq * Hq].view(Mq, Hq)))
    # the consumer side, timed last (its allocations perturbed the GEMM
    # timings when it ran before them): the fused GEMM hands downstream code
    # column slices that keep the fused row stride, split projections are
    # contiguous.  A per-row RMS norm of q and k (torch's rms_norm, standing
    # in for the downstream QK norm; not a step of this path) on both
    if hasattr(torch.nn.functional, "rms_norm"):
        rms, nw = torch.nn.functional.rms_norm, torch.ones(Hq, dtype=torch.bfloat16, device=dev)
        qs, ks = ycat[:, :Hq], ycat[:, Hq:2 * Hq]
        out["consumer_qk_rmsnorm_contiguous_us"] = timed(lambda: (rms(ys[0], (Hq,), nw), rms(ys[1], (Hq,), nw)))
        out["consumer_qk_rmsnorm_strided_us"] = timed(lambda: (rms(qs, (Hq,), nw), rms(ks, (Hq,), nw)))
    del qa, ws, ys, wcat, ycat, xq, wsq
    torch.cuda.empty_cache()
    return out


def single_linear(fp8, torch, dev, stream, workloads):
    """The single-Linear workload (X [64, 512] with outliers, W [512, 512],
    per-tensor static scales): quantize + one GEMM, 33.6 MFLOP over ~0.4 MB,
    a latency-bound call.  Back-to-back eager calls (the binding's host cost
    included) and each kernel alone; HIP graphs holding one call, 50 calls,
    50 quantizations and 50 GEMMs, whose replays give the GPU time per call
    with one graph launch spread over 100 kernels (each graph's output
    checked against the eager one, synchronizing between replays)."""
    wl = workloads.single_linear()
    x = dev_bf16(torch, wl.x, dev)
    qw, sw = fp8.rtn_weight(dev_bf16(torch, wl.weights["w"], dev))
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe(x, st, fp8.OBS_MAX)
    sx = fp8.fp8_scale_from_state(st)
    M, K = x.shape
    N = qw.shape[0]
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def call():
        fp8.fp8_quant_static(x, sx, out=qx)
        fp8.fp8_linear(qx, qw, sx, sw, out=y)

    flops = 2.0 * M * N * K
    out = {"workload": wl.name, "flops": flops}
    out["eager_call_us"] = time_launches(torch, stream, lambda r: call(), 500, warm=20)
    out["quant_us"] = time_launches(torch, stream, lambda r: fp8.fp8_quant_static(x, sx, out=qx), 500, warm=20)
    out["gemm_us"] = time_launches(torch, stream, lambda r: fp8.fp8_linear(qx, qw, sx, sw, out=y), 500, warm=20)
    call()
    torch.cuda.synchronize()
    ref = y.clone()

    def graph_of(fn, n):
        side = torch.cuda.Stream(device=dev)   # warm-up on a side stream before capture
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        return g

    quant = lambda: fp8.fp8_quant_static(x, sx, out=qx)        # noqa: E731
    gemm = lambda: fp8.fp8_linear(qx, qw, sx, sw, out=y)        # noqa: E731
    graphs = {"one_call": graph_of(call, 1), "calls": graph_of(call, 50),
              "quant": graph_of(quant, 50), "gemm": graph_of(gemm, 50)}
    for name in ("one_call", "calls", "gemm"):
        for _ in range(3):
            y.zero_()
            torch.cuda.synchronize()
            graphs[name].replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"{name} graph differs"
    t = {k: time_launches(torch, stream, lambda r, g=g: g.replay(), 100, warm=5) for k, g in graphs.items()}
    out["graph_one_call_us"] = t["one_call"]
    # GPU time: 50 calls (100 launches) captured in one graph, per call
    out["gpu_call_us"] = t["calls"] / 50
    out["gpu_quant_us"] = t["quant"] / 50
    out["gpu_gemm_us"] = t["gemm"] / 50
    out["gpu_TFLOP/s"] = tflops(flops, out["gpu_call_us"])
    out["note"] = ("latency-bound: eager calls are bound by the host (two library calls); a graph "
                   "holding one call costs more to launch than the two eager launches it replaces; "
                   "gpu_* are per call from 50 calls captured in one graph")
    del graphs
    return out


def per_row_fp8(fp8, torch, dev, stream):
    """Per-row FP8 (per-token activation / per-channel weight scales) beside
    the per-tensor path: per-token quantization of X [2048, 2048] and of
    X [16384, 5120] (3 B per element), and a [2048, 8192, 2048] projection
    with per-row scales on both engines (TFLOP/s)."""
    def timed(f, reps):
        return time_launches(torch, stream, f, reps, warm=2)

    out = {}
    for rows, k, reps in ((2048, 2048, 50), (16384, 5120, 20)):
        xs = [torch.randn((rows, k), device=dev).to(torch.bfloat16) for _ in range(3)]
        q = torch.empty((rows, k), dtype=torch.uint8, device=dev)
        sc = torch.empty(rows, dtype=torch.float32, device=dev)
        us = timed(lambda r: fp8.fp8_quant_per_row(xs[r % 3], out=q, scales=sc), reps)
        out[f"quant_per_row_{rows}x{k}"] = {"us": us, "bytes": 3 * rows * k,
                                            "GB/s": 3 * rows * k / us / 1e3,
                                            "frac_hbm": 3 * rows * k / us / 1e3 / HBM_PEAK_GBS}
        del xs, q, sc
    M, H, I = 2048, 2048, 8192
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


def two_tower_layer(fp8, torch, dev, stream):
    """One decoder layer's FP8 Linear set for both towers (H=4096, I=12288;
    und M=512 tokens, gen M=4096): per tower qkv_fp8 (one quantization, three
    GEMMs), the o projection (its own quantize + GEMM) and gated_mlp_fp8, on
    the seeded forward inputs, under each of the two static scale sets the
    library's observers produce from the 256 seeded calibration calls (max
    observer; moving average of the per-call maxima, constant 0.01).
    Weights N(0, 0.02) RTN per tensor on the GPU.  Average time of the whole
    set under each scale set, both engines (FP8 engine flagged)."""
    from mlp_fp8_quant_amd import calibration, workloads
    H, I = workloads.LAYER_H, workloads.LAYER_I
    towers = {}
    for name, M in workloads.TOWER_M.items():
        t = {"M": M}
        t["scales"] = calibration.calibrate_tower(name, dev)
        for k, w in workloads.layer_weights(name).items():
            t["w_" + k], t["s_" + k] = fp8.rtn_weight(dev_bf16(torch, w, dev))
        for site in ("qkv", "o", "gateup"):
            t["x_" + site] = dev_bf16(torch, workloads.forward_input(name, site), dev)
        t["outs"] = tuple(torch.empty((M, H), dtype=torch.bfloat16, device=dev) for _ in range(3))
        t["ws_qkv"] = torch.empty(fp8.qkv_fp8_workspace(M, H), dtype=torch.uint8, device=dev)
        t["qo"] = torch.empty((M, H), dtype=torch.uint8, device=dev)
        t["yo"] = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        t["ws_mlp"] = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8,
                                  device=dev)
        t["y"] = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        t["flops"] = 2.0 * M * H * H * 4 + 3 * 2.0 * M * I * H
        towers[name] = t

    def layer(t, sc, acc):
        fp8.qkv_fp8(t["x_qkv"], sc["qkv"], t["w_q"], t["s_q"], t["w_k"], t["s_k"],
                    t["w_v"], t["s_v"], outs=t["outs"], workspace=t["ws_qkv"], accum=acc)
        fp8.fp8_quant_static(t["x_o"], sc["o"], out=t["qo"])
        fp8.fp8_linear(t["qo"], t["w_o"], sc["o"], t["s_o"], out=t["yo"], accum=acc)
        fp8.gated_mlp_fp8(t["x_gateup"], sc["gateup"], t["w_gate"], t["s_gate"], t["w_up"],
                          t["s_up"], sc["down"], t["w_down"], t["s_down"], out=t["y"],
                          workspace=t["ws_mlp"], accum=acc)

    def timed(f, reps=20):
        return time_launches(torch, stream, lambda r: f(), reps, warm=5)

    out = {"workload": "two_tower_layer_H4096_I12288_und512_gen4096",
           "gemm_flops": {k: t["flops"] for k, t in towers.items()},
           "scales": {k: {("max" if mode == fp8.OBS_MAX else "moving_avg"):
                          {site: float(v.item()) for site, v in sc.items()}
                          for mode, sc in t["scales"].items()}
                      for k, t in towers.items()}}
    for set_name, mode in (("max", fp8.OBS_MAX), ("moving_avg", fp8.OBS_MOVING_AVG)):
        for en, acc in (("exact", fp8.ACC_EXACT), ("fp8_mfma", fp8.ACC_FP8_MFMA)):
            r = {}
            for k, t in towers.items():
                us = timed(lambda: layer(t, t["scales"][mode], acc))
                r[k] = {"us": us, "TFLOP/s": t["flops"] / (us * 1e-6) / 1e12}
            us = timed(lambda: [layer(t, t["scales"][mode], acc) for t in towers.values()])
            tot = sum(t["flops"] for t in towers.values())
            r["both_towers"] = {"us": us, "TFLOP/s": tot / (us * 1e-6) / 1e12,
                                "frac_fp8_peak": tot / (us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS}
            if acc == fp8.ACC_FP8_MFMA:
                r.update(meets_tolerance=False, note=FP8_ENGINE_NOTE)
            out[f"{set_name}_{en}"] = r
    del towers
    torch.cuda.empty_cache()
    return out


def elementwise_large(fp8, torch, dev, stream):
    """The HBM-bound kernels at the large gated-MLP sizes (X [16384, 5120],
    G/U [16384, 25600], or G|U adjacent in one [16384, 51200] tensor for the
    one-input SwiGLU), where the working sets exceed the 256 MB MALL:
    average launch time over back-to-back launches (three rotating X copies
    for quantize), algorithmic GB/s and the fraction of the 8 TB/s peak,
    beside the read/write ceiling of the same byte mix (the library's
    no-arithmetic kernel with the same access pattern and grid; kernel and
    ceiling timed alternately three times, medians) and a plain device copy."""
    def timed(f, reps):
        return time_launches(torch, stream, f, reps, warm=2)

    def against_ceiling(kernel, ceiling, reps, rounds=3):
        # kernel and ceiling timed alternately, `rounds` times each; medians
        ks, cs = [], []
        for _ in range(rounds):
            ks.append(timed(kernel, reps))
            cs.append(timed(ceiling, reps))
        return sorted(ks)[rounds // 2], sorted(cs)[rounds // 2]

    out = {}
    n = 16384 * 5120
    xs = [torch.randn(n, device=dev).to(torch.bfloat16) for _ in range(3)]
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    s = torch.tensor([0.02], device=dev)
    us, uc = against_ceiling(lambda r: fp8.fp8_quant_static(xs[r % 3], s, out=q),
                             lambda r: fp8.rw_ceiling(xs[r % 3], None, q), 20)
    out["quant_16384x5120"] = {"us": us, "bytes": 3 * n, "GB/s": 3 * n / us / 1e3,
                               "frac_hbm": 3 * n / us / 1e3 / HBM_PEAK_GBS,
                               "ceiling_us": uc, "ceiling_GB/s": 3 * n / uc / 1e3}
    del xs, q
    n = 16384 * 25600
    g = torch.randn(n, device=dev).to(torch.bfloat16)
    u = torch.randn(n, device=dev).to(torch.bfloat16)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    us, uc = against_ceiling(lambda r: fp8.silu_mul_2in_fp8(g, u, s, out=q),
                             lambda r: fp8.rw_ceiling(g, u, q), 8)
    out["silu_16384x25600"] = {"us": us, "bytes": 5 * n, "GB/s": 5 * n / us / 1e3,
                               "frac_hbm": 5 * n / us / 1e3 / HBM_PEAK_GBS,
                               "ceiling_us": uc, "ceiling_GB/s": 5 * n / uc / 1e3}
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


def code_digest(path):
    """sha256[:16] of a HIP source's code: its // comments and all white
    space left out, so that a comment edit keeps a counter record valid and
    any change to the code invalidates it."""
    import hashlib
    import re
    words = []
    for line in open(path, encoding="utf-8"):
        words.extend(re.sub(r"//.*", "", line).split())
    return hashlib.sha256(" ".join(words).encode()).hexdigest()[:16]


def recorded_traffic(key, source):
    """HBM-side bytes per launch of a kernel, as recorded from rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by a plain copy of known size) in
    profiles/traffic.md, or None when that record is missing or was taken
    from a different version of the kernel's source file."""
    path = os.path.join(ROOT, "profiles", "traffic.md")
    src = os.path.join(ROOT, "mlp_fp8_quant_amd", "csrc", source)
    try:
        digest = code_digest(src)
        for line in open(path):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 5 and cells[0] == key and cells[4] == digest:
                return {"fetch_bytes": float(cells[1]), "write_bytes": float(cells[2]),
                        "total_bytes": float(cells[1]) + float(cells[2]),
                        "algorithmic_bytes": float(cells[3])}
    except (OSError, ValueError):
        pass
    return None


def cpu_baseline(wl, rows, channels):
    """The oracle, as it stands, on a bounded block of the same workload:
    rows 0..rows-1 of X and intermediate channels 0..channels-1 (those rows
    of W_gate and W_up, those columns of W_down, RTN-quantized with their
    whole tensors' scales beforehand, as weights are at load) through the
    whole chain: quantize X, exact gate/up GEMMs with the BF16 epilogue, the
    down input scale from silu(G)*U, FP8 SwiGLU, exact down GEMM with the
    BF16 epilogue.  Reported in the metric's unit: GEMM TFLOP/s of the
    block."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import linear as olin
    from oracle.swiglu import silu_mul_f64, silu_mul_fp8

    x = wl.x[:rows]
    C = channels
    wq = {"gate": wl.weights["gate"][:C], "up": wl.weights["up"][:C],
          "down": np.ascontiguousarray(wl.weights["down"][:, :C])}
    q, s = {}, {}
    for k in wq:
        s[k] = olin.scale_from_amax(olin.amax_f32(wl.weights[k]))
        q[k] = olin.quant_static(wq[k], s[k])
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
    flops = 2.0 * rows * C * H * 3
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": dt, "cpu_model": cpu_model,
            "sample": f"rows 0..{rows - 1} of X [{wl.x.shape[0]}, {H}] x intermediate "
                      f"channels 0..{C - 1} of {wl.weights['gate'].shape[0]} through the whole "
                      f"gated MLP ({flops / 1e9:.0f} GFLOP); float64 exact GEMMs, "
                      f"os.cpu_count()={os.cpu_count()}"}


if __name__ == "__main__":
    main()
