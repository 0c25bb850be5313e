"""Pins for oracle.swiglu and oracle.observer."""

import numpy as np
import torch

from oracle.formats import bf16_to_f32, e4m3_encode
from oracle.linear import scale_from_amax
from oracle.observer import (OBS_MAX, OBS_MOVING_AVG, ObserverState,
                             calibrate, call_amax, observe)
from oracle.swiglu import silu_mul_f64, silu_mul_fp8
from mlp_fp8_quant_amd import workloads


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def torch_e4m3(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_silu_mul_against_torch_silu():
    rng = np.random.default_rng(11)
    g = _bf16(rng.standard_normal(200_000) * 4)
    u = _bf16(rng.standard_normal(200_000) * 3)
    s = np.float32(0.371)
    ours = silu_mul_fp8(g, u, s)
    g64 = torch.from_numpy(bf16_to_f32(g).astype(np.float64))
    u64 = torch.from_numpy(bf16_to_f32(u).astype(np.float64))
    h = torch.nn.functional.silu(g64) * u64
    q = (h / float(s)).to(torch.float32).numpy()
    inr = np.abs(q) <= 464
    assert inr.mean() > 0.99
    assert np.array_equal(ours[inr], torch_e4m3(q[inr]))
    assert np.all((ours[~inr] & 0x7F) == 0x7E)


def test_silu_mul_special_cases():
    s = np.float32(0.05)
    # g = +-0: silu is a signed zero, the code is +-0 with the product's sign
    g = _bf16([0.0, 0.0, -0.0, -0.0])
    u = _bf16([2.0, -2.0, 2.0, -2.0])
    assert list(silu_mul_fp8(g, u, s)) == [0x00, 0x80, 0x80, 0x00]
    # g >= 40: 1 + exp(-g) == 1 in float64, so h = g*u exactly
    g = _bf16([40.0, 64.0, 100.0])
    u = _bf16([0.25, -0.125, 1e-3])
    gu = bf16_to_f32(g).astype(np.float64) * bf16_to_f32(u).astype(np.float64)
    assert np.array_equal(silu_mul_fp8(g, u, s),
                          e4m3_encode((gu / np.float64(s)).astype(np.float32)))
    # very negative g: exp(-g) overflows, silu -> -0
    g = _bf16([-1e4, -3e38])
    u = _bf16([1.0, -1.0])
    assert list(silu_mul_fp8(g, u, s)) == [0x80, 0x00]
    assert np.all(silu_mul_f64(g, u) == 0)


def test_call_amax_matches_integer_definition():
    rng = np.random.default_rng(12)
    x = _bf16(rng.standard_normal(100_000) * 7)
    a = call_amax(x)
    m = int(np.max(x & 0x7FFF))
    assert a == bf16_to_f32(np.array([m], np.uint16))[0]
    x[5] = 0x7FC1  # a NaN propagates
    assert np.isnan(call_amax(x))


def test_max_observer_is_running_max():
    vals = [3.0, 7.5, 2.0, 7.5, 9.25, 1.0]
    st = ObserverState()
    for v in vals:
        observe(st, v, OBS_MAX)
    assert st.m == np.float32(9.25) and st.count == 6


def test_moving_average_closed_forms():
    # constant input: m + c*(a - m) = m exactly
    st = ObserverState()
    for _ in range(300):
        observe(st, 5.5, OBS_MOVING_AVG, 0.01)
    assert st.m == np.float32(5.5)
    # c = 1 keeps the last value when consecutive values are within a factor
    # of 2 (a - m and m + (a - m) are then exact by Sterbenz' lemma)
    st = ObserverState()
    for v in (3.0, 4.5, 2.5, 3.75):
        observe(st, v, OBS_MOVING_AVG, 1.0)
        assert st.m == np.float32(v)
    # first call initializes the state
    st = ObserverState()
    observe(st, 12.0, OBS_MOVING_AVG, 0.01)
    assert st.m == np.float32(12.0)


def test_moving_average_against_float64_recurrence_and_bounds():
    rng = np.random.default_rng(13)
    a = rng.uniform(5.0, 30.0, 256).astype(np.float32)
    st = ObserverState()
    exact = None
    c64 = float(np.float32(0.01))
    for v in a:
        observe(st, v, OBS_MOVING_AVG, 0.01)
        exact = float(v) if exact is None else exact + c64 * (float(v) - exact)
    # each step adds at most ~3 float32 roundings of magnitude <= 30
    assert abs(float(st.m) - exact) <= 256 * 3 * 30 * 2.0 ** -24
    assert a.min() <= st.m <= a.max()


def test_moving_average_clips_below_max_on_spiky_calls():
    # two-tower calibration recipe at reduced size: the MA scale sits below
    # the max-observer scale and a forward draw saturates under it
    base = workloads.calib_base("und", "qkv", rows=64)
    calls = []
    for t in range(256):
        pos, gain = workloads.calib_spikes("und", "qkv", t, base.size)
        calls.append(workloads.calib_call(base, pos, gain))
    s_max = calibrate(calls, OBS_MAX)
    s_ma = calibrate(calls, OBS_MOVING_AVG, 0.01)
    assert s_ma < s_max
    amaxes = np.array([call_amax(c) for c in calls])
    assert s_max == scale_from_amax(amaxes.max())
    x = calls[int(np.argmax(amaxes))]  # the spikiest call clips under MA
    from oracle.linear import quant_static
    q = quant_static(x, s_ma)
    assert np.count_nonzero((q & 0x7F) == 0x7E) > 0


def test_observer_constants_are_the_printed_ones():
    # the averaging constant and the calibration length the model card prints
    # (tests/golden, cited there) are the oracle's defaults, the library's
    # calibration constant and the seeded calibration recipe's length
    import inspect
    import json
    import os
    from mlp_fp8_quant_amd import calibration
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "pages_printed_values.json")))["observer"]
    c = g["averaging_constant"]
    for f in (observe, calibrate):
        assert inspect.signature(f).parameters["c"].default == c
    assert float(calibration.MA_CONSTANT) == c
    assert workloads.CALIB_CALLS == g["calibration_calls"]
