"""Activation observers that produce the static input scales.

Model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN ...": the plain RTN build
takes each static input scale from the global max of the activations seen
during calibration; the card's checkpoint instead keeps a moving average of the per-call
maxima (MOVING_AVERAGE_MINMAX, averaging constant 0.01), which clips the
rarest activations (header paragraph and section "Scheme").  Calibration ran
256 transformer calls.

Readings (pages silent): the quantity averaged is the per-call amax
max|x|; the first call initializes the state (m_1 = a_1); the update is
m_t = m_{t-1} + c * (a_t - m_{t-1}) with c = fp32(0.01) and three separately
rounded float32 operations (subtract, multiply, add; no fused multiply-add);
the scale is fp32(m / 448).  A NaN amax propagates into the state.
"""

import numpy as np

from .formats import bf16_to_f32
from .linear import scale_from_amax

OBS_MAX = 0
OBS_MOVING_AVG = 1


class ObserverState:
    """Running state: m (float32) and the number of calls seen."""

    def __init__(self):
        self.m = np.float32(0.0)
        self.count = 0


def call_amax(x_bf16) -> np.float32:
    """Per-call amax = max |x| as float32; NaN if any element is NaN."""
    x = bf16_to_f32(x_bf16)
    if x.size == 0:
        return np.float32(0.0)
    a = np.abs(x)
    if np.any(np.isnan(a)):
        return np.float32(np.nan)
    return np.float32(a.max())


def observe(state: ObserverState, a, mode: int, c=0.01) -> ObserverState:
    """Fold one per-call amax ``a`` into the state."""
    a = np.float32(a)
    c = np.float32(c)
    if state.count == 0:
        m = a
    elif mode == OBS_MAX:
        m = a if (np.isnan(a) or np.isnan(state.m)) else max(state.m, a)
        m = np.float32(m)
    elif mode == OBS_MOVING_AVG:
        d = np.float32(a - state.m)
        p = np.float32(c * d)
        m = np.float32(state.m + p)
    else:
        raise ValueError("unknown observer mode")
    state.m = np.float32(m)
    state.count += 1
    return state


def calibrate(calls, mode: int, c=0.01) -> np.float32:
    """Run the observer over a sequence of BF16 tensors; return the scale."""
    st = ObserverState()
    for x in calls:
        observe(st, call_amax(x), mode, c)
    return scale_from_amax(st.m)
