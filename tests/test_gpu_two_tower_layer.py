"""GPU parity of the two-tower decoder layer's FP8 Linear set (H = 4096,
I = 12288; und tower 512 tokens, gen tower 4096) under the static input
scales of its 256 calibration calls, computed both ways (model card
"Cosmos3-Nano-Policy-DROID, FP8 + RTN + moving-average activation
observer", header paragraph and "Scheme": the max observer, and a moving
average of the per-call maxima with constant 0.01).

* Calibration: the gen tower's 256 calls at all four observer sites (inputs
  of q/k/v, o, gate/up and down), both observers, bit-exact.  The GPU folds
  every materialized call (mlp_fp8_quant_amd.calibration); the oracle folds
  each call's amax, taken as max(amax(base), max |spike values|): a spike
  multiplies an entry by a gain >= 5, so no spiked entry falls below its
  base value and the two agree (checked against the oracle's amax of fully
  materialized calls in test_workloads_cpu.py).  (The und tower's 256
  calls are in test_gpu_quant_observer.py.)
* The layer, per tower and per scale set: qkv_fp8, the o projection
  (fp8_quant_static + fp8_linear) and gated_mlp_fp8 (down input scale = the
  calibrated down-site scale) on the forward inputs.  Weights RTN on the GPU
  equal the oracle's; qX codes at every site are bit-exact (the workspaces
  hold them); the moving-average set saturates the gate/up input of each
  tower (its forward amax exceeds the average) while the max set does not;
  q/k/v/o outputs and the gated MLP's qH and y on sampled rows (all 512 of
  the und tower, 64 of the gen tower) against the oracle stage by stage, and
  y against the whole oracle chain with the bound widened by exactly the
  SwiGLU codes that differ by one step.
"""

import functools

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import calibration, workloads
from oracle import linear as olin
from oracle import observer as oobs
from oracle.formats import e4m3_decode
from oracle.swiglu import silu_mul_fp8

from gpu_util import (check_fp8_tolerance, check_gemm_bf16, device, host_bits,
                      host_f32, host_u8, oracle_quant_threaded, oracle_rtn_threaded,
                      report, scalar, to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu

MODES = {"max": fp8.OBS_MAX, "ma": fp8.OBS_MOVING_AVG}
H, I = workloads.LAYER_H, workloads.LAYER_I


def _call_amaxes(tower, site):
    """Oracle per-call amax of the site's 256 calibration calls."""
    base = workloads.calib_base(tower, site)
    a_base = oobs.call_amax(base)
    out = []
    for t in range(workloads.CALIB_CALLS):
        pos, gain = workloads.calib_spikes(tower, site, t, base.size)
        vals = workloads.calib_spike_values(base, pos, gain)
        out.append(np.float32(max(a_base, oobs.call_amax(vals))))
    return out


@functools.lru_cache(maxsize=None)
def _oracle_states(tower):
    """{mode name: {site: ObserverState}} from the oracle's fold."""
    res = {k: {} for k in MODES}
    for site in workloads.SITES:
        amaxes = _call_amaxes(tower, site)
        for k, mode in MODES.items():
            st = oobs.ObserverState()
            for a in amaxes:
                oobs.observe(st, a, mode, 0.01)
            res[k][site] = st
    return res


def test_gen_tower_calibration_all_sites_both_observers():
    dev = device()
    want = _oracle_states("gen")
    for site in workloads.SITES:
        print(f"gen tower calibration site={site}", flush=True)
        states = calibration.calibrate_site("gen", site, dev)
        for k, mode in MODES.items():
            a = states[mode].cpu().numpy()
            m = a[:1].view(np.float32)[0]
            assert int(a[1]) == workloads.CALIB_CALLS and int(a[2]) == 0 and int(a[3]) == 0
            assert m.view(np.uint32) == np.float32(want[k][site].m).view(np.uint32), (site, k)
            s = host_f32(fp8.fp8_scale_from_state(states[mode]))[0]
            assert s == olin.scale_from_amax(want[k][site].m), (site, k)


def _chained_bound_check(y_bits, qh_gpu, qh_oracle, S, A, alpha, qw_down):
    """y against the oracle chain: |y - alpha S| <= alpha (sum_k |dqH| |qWd|
    + 1e-5 sum|terms|) + 1 BF16 ulp, S and A the oracle chain's sums."""
    dH = np.abs(e4m3_decode(qh_gpu) - e4m3_decode(qh_oracle))
    extra = dH @ np.abs(e4m3_decode(qw_down)).T
    yf = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.float64(alpha) * S
    bound = np.float64(alpha) * (extra + 1e-5 * A) + np.abs(ref) * 2.0 ** -7 + 1e-300
    assert np.all(np.abs(yf - ref) <= bound)


@pytest.mark.parametrize("tower", ["und", "gen"])
def test_layer_under_both_calibrated_scale_sets(tower):
    dev = device()
    M = workloads.TOWER_M[tower]
    rows = (np.arange(M) if M <= 512 else
            np.sort(np.random.default_rng(23).choice(M, 64, replace=False)))
    drows = torch.from_numpy(rows).to(dev)
    print(f"layer {tower}: weights", flush=True)
    wts = workloads.layer_weights(tower)
    dq, ds, oq, os_ = {}, {}, {}, {}
    for p, w in wts.items():
        dq[p], ds[p] = fp8.rtn_weight(to_dev_bf16(w, dev))
        oq[p], os_[p] = oracle_rtn_threaded(w)
        assert host_f32(ds[p])[0] == os_[p], p
        assert np.array_equal(host_u8(dq[p]), oq[p]), p
    del wts
    xs = {site: workloads.forward_input(tower, site) for site in ("qkv", "o", "gateup")}
    dxs = {site: to_dev_bf16(x, dev) for site, x in xs.items()}
    states = _oracle_states(tower)
    for k in MODES:
        print(f"layer {tower}: scale set {k}", flush=True)
        sc = {site: olin.scale_from_amax(states[k][site].m) for site in workloads.SITES}
        dsc = {site: scalar(v, dev) for site, v in sc.items()}
        # q/k/v over one shared quantization
        ws_qkv = torch.empty(fp8.qkv_fp8_workspace(M, H), dtype=torch.uint8, device=dev)
        yq, yk, yv = fp8.qkv_fp8(dxs["qkv"], dsc["qkv"], dq["q"], ds["q"], dq["k"], ds["k"],
                                 dq["v"], ds["v"], workspace=ws_qkv)
        # o projection: its own quantization and GEMM
        qo = fp8.fp8_quant_static(dxs["o"], dsc["o"])
        yo = fp8.fp8_linear(qo, dq["o"], dsc["o"], ds["o"])
        # gated MLP, down input scale = the calibrated down-site scale
        ws_mlp = torch.empty(fp8.gated_mlp_fp8_workspace(M, H, I), dtype=torch.uint8, device=dev)
        y = fp8.gated_mlp_fp8(dxs["gateup"], dsc["gateup"], dq["gate"], ds["gate"], dq["up"],
                              ds["up"], dsc["down"], dq["down"], ds["down"], workspace=ws_mlp)
        torch.cuda.synchronize()
        # qX at every site, bit-exact (the composites' workspaces hold them)
        qx = {"qkv": host_u8(ws_qkv[:M * H]).reshape(M, H), "o": host_u8(qo),
              "gateup": host_u8(ws_mlp[:M * H]).reshape(M, H)}
        for site, q in qx.items():
            assert np.array_equal(q, oracle_quant_threaded(xs[site], sc[site])), (site, k)
        sat = {site: int(np.count_nonzero((q & 0x7F) == 0x7E)) for site, q in qx.items()}
        report(f"two_tower_{tower}_{k}_saturated_codes", sat)
        if k == "ma":
            assert sat["gateup"] > 0       # the moving average clips the rarest spikes
        else:
            assert sum(sat.values()) == 0  # the max set holds every forward value
        # q/k/v and o on the sampled rows (BF16 per R-13)
        for p, t, site in (("q", yq, "qkv"), ("k", yk, "qkv"), ("v", yv, "qkv"), ("o", yo, "o")):
            dqx = torch.from_numpy(qx[site]).to(dev)
            y32 = host_f32(fp8.fp8_linear(dqx, dq[p], dsc[site], ds[p], fp8.OUT_F32)[drows])
            S, A = olin.gemm_exact(qx[site][rows], oq[p])
            n2 = check_gemm_bf16(host_bits(t[drows]), y32, S, A, olin.epilogue_alpha(sc[site], os_[p]))
            report(f"two_tower_{tower}_{k}_{p}_r13_second_clause", n2)
        # gated MLP: qH (SwiGLU bar against the oracle's G, U), then y
        l_qh = M * H   # qX [M, H] is 256-byte aligned at these sizes
        qh = host_u8(ws_mlp[l_qh:l_qh + M * I]).reshape(M, I)[rows]
        Sg, _ = olin.gemm_exact(qx["gateup"][rows], oq["gate"])
        Su, _ = olin.gemm_exact(qx["gateup"][rows], oq["up"])
        G = olin.epilogue_bf16(Sg, sc["gateup"], os_["gate"])
        U = olin.epilogue_bf16(Su, sc["gateup"], os_["up"])
        qh_o = silu_mul_fp8(G, U, sc["down"]).reshape(rows.size, I)
        n_off = check_fp8_tolerance(qh.ravel(), qh_o.ravel())
        report(f"two_tower_{tower}_{k}_swiglu_codes_one_step_off_frac", n_off / qh.size)
        report(f"two_tower_{tower}_{k}_qh_saturated_codes",
               int(np.count_nonzero((qh & 0x7F) == 0x7E)))
        # stage-wise: the down GEMM on the GPU's own qH rows
        dqh = ws_mlp[l_qh:l_qh + M * I].view(M, I)
        y32 = host_f32(fp8.fp8_linear(dqh, dq["down"], dsc["down"], ds["down"], fp8.OUT_F32)[drows])
        S, A = olin.gemm_exact(qh, oq["down"])
        alpha_d = olin.epilogue_alpha(sc["down"], os_["down"])
        n2 = check_gemm_bf16(host_bits(y[drows]), y32, S, A, alpha_d)
        report(f"two_tower_{tower}_{k}_down_r13_second_clause", n2)
        # chained: against the oracle's own qH
        So, Ao = olin.gemm_exact(qh_o, oq["down"])
        _chained_bound_check(host_bits(y[drows]), qh, qh_o, So, Ao, alpha_d, oq["down"])
        del ws_qkv, ws_mlp, yq, yk, yv, qo, yo, y
    torch.cuda.empty_cache()
