"""Static input scales of the two-tower decoder layer from its calibration
calls, through the library's observer (model card "Cosmos3-Nano-Policy-DROID,
FP8 + RTN + moving-average activation observer", header paragraph and
"Scheme": static input scales from the global maximum of the activations
over the calibration calls, or from a moving average of the per-call maxima
with constant 0.01).

Each observer site (the input of q/k/v, of o, of gate/up and of down) sees
the seeded calibration calls of ``workloads``: a fixed base tensor with a
fresh set of spikes per call.  Every call is materialized on the GPU (the
base, with the call's spike values written at their positions) and folded
into both observers, so one pass gives both scale sets.
"""

import torch

from . import workloads
from .api import (OBS_MAX, OBS_MOVING_AVG, fp8_observe, fp8_scale_from_state,
                  new_observer_state)

MA_CONSTANT = 0.01


def _bf16(bits, device):
    return torch.from_numpy(bits.view("int16")).view(torch.bfloat16).to(device)


def calibrate_site(tower, site, device, calls=workloads.CALIB_CALLS, c=MA_CONSTANT):
    """Observer states {OBS_MAX: state, OBS_MOVING_AVG: state} of one site
    after `calls` calibration calls."""
    base = workloads.calib_base(tower, site)
    dbase = _bf16(base, device).view(-1)
    work = torch.empty_like(dbase)
    states = {OBS_MAX: new_observer_state(device), OBS_MOVING_AVG: new_observer_state(device)}
    for t in range(calls):
        pos, gain = workloads.calib_spikes(tower, site, t, base.size)
        vals = workloads.calib_spike_values(base, pos, gain)
        work.copy_(dbase)
        work[torch.from_numpy(pos).to(device)] = _bf16(vals, device)
        fp8_observe(work, states[OBS_MAX], OBS_MAX)
        fp8_observe(work, states[OBS_MOVING_AVG], OBS_MOVING_AVG, c)
    return states


def calibrate_tower(tower, device, calls=workloads.CALIB_CALLS, c=MA_CONSTANT):
    """Both scale sets of one tower: {mode: {site: scale}}, each scale a
    one-element float32 device tensor (state.m / 448)."""
    out = {OBS_MAX: {}, OBS_MOVING_AVG: {}}
    for site in workloads.SITES:
        st = calibrate_site(tower, site, device, calls, c)
        for mode, state in st.items():
            out[mode][site] = fp8_scale_from_state(state)
    return out
