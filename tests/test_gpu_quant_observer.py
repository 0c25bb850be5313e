"""GPU parity: static quantization, RTN weights and the observers, bit-exact
against the oracle."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin
from oracle import observer as oobs

from gpu_util import device, host_f32, host_u8, scalar, to_dev_bf16

pytestmark = pytest.mark.gpu

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 2.0 ** 5, 0.0123, 20.0 / 448,
                                   3.7e-3, 1.337, 1e-30, 7.5e30])
def test_quant_exhaustive_bf16(scale):
    dev = device()
    s = np.float32(scale)
    q = fp8.fp8_quant_static(to_dev_bf16(ALL_BF16, dev), scalar(s, dev))
    assert np.array_equal(host_u8(q), olin.quant_static(ALL_BF16, s))


def test_quant_exhaustive_random_scales():
    dev = device()
    x = to_dev_bf16(ALL_BF16, dev)
    rng = np.random.default_rng(20)
    for s in np.exp(rng.uniform(-12, 8, 16)).astype(np.float32):
        q = fp8.fp8_quant_static(x, scalar(s, dev))
        assert np.array_equal(host_u8(q), olin.quant_static(ALL_BF16, s)), s


@pytest.mark.parametrize("m", [1.0, 3.0, 0.0123])
def test_quant_exhaustive_scales_next_to_exact(m):
    # s = m * (1 + k 2^-23): x / s lands within a few FP32 units of the E4M3
    # rounding boundaries that BF16 inputs sit on exactly (every midpoint
    # has 5 significant bits), where a quotient taken through 1/s can round
    # the other way; the codes must still be those of the IEEE quotient
    dev = device()
    x = to_dev_bf16(ALL_BF16, dev)
    for k in range(-6, 7):
        s = np.float32(m) * np.float32(1.0 + k * 2.0 ** -23)
        q = fp8.fp8_quant_static(x, scalar(s, dev))
        assert np.array_equal(host_u8(q), olin.quant_static(ALL_BF16, s)), (m, k)


@pytest.mark.parametrize("scale", [1e-39, 3e38, 2.0 ** -126, 2.0 ** 126])
def test_quant_exhaustive_extreme_scales(scale):
    # 1/s subnormal or infinite: every element takes the IEEE division
    dev = device()
    s = np.float32(scale)
    q = fp8.fp8_quant_static(to_dev_bf16(ALL_BF16, dev), scalar(s, dev))
    assert np.array_equal(host_u8(q), olin.quant_static(ALL_BF16, s))


@pytest.mark.parametrize("n", [0, 1, 7, 15, 16, 17, 255, 4097, 1_000_003])
def test_quant_ragged_lengths(n):
    dev = device()
    rng = np.random.default_rng(n)
    bits = rng.integers(0, 65536, n, dtype=np.int64).astype(np.uint16)
    s = np.float32(0.031)
    q = fp8.fp8_quant_static(to_dev_bf16(bits, dev), scalar(s, dev))
    assert np.array_equal(host_u8(q), olin.quant_static(bits, s))


@pytest.mark.parametrize("name", ["single_linear", "gen_mlp", "split_qkv"])
def test_quant_config_activations(name):
    dev = device()
    wl = workloads.CONFIGS[name]()
    s = olin.scale_from_amax(olin.amax_f32(wl.x))
    q = fp8.fp8_quant_static(to_dev_bf16(wl.x, dev), scalar(s, dev))
    assert np.array_equal(host_u8(q), olin.quant_static(wl.x, s))


def test_quant_super_mlp_activation_sampled():
    # 16384 x 5120: every code checked on a seeded sample of 4M positions
    dev = device()
    rng = np.random.default_rng(0)
    x = workloads.activations(rng, 16384, 5120, outliers=True)
    s = olin.scale_from_amax(olin.amax_f32(x))
    q = host_u8(fp8.fp8_quant_static(to_dev_bf16(x, dev), scalar(s, dev))).ravel()
    pos = np.random.default_rng(1).choice(x.size, 4_000_000, replace=False)
    assert np.array_equal(q[pos], olin.quant_static(x.ravel()[pos], s))


@pytest.mark.parametrize("name", ["single_linear", "gen_mlp"])
def test_rtn_weights_on_gpu_match_oracle(name):
    dev = device()
    wl = workloads.CONFIGS[name]()
    for w in wl.weights.values():
        q, s = fp8.rtn_weight(to_dev_bf16(w, dev))
        oq, os_ = olin.rtn_weight(w)
        assert host_f32(s)[0].view(np.uint32) == np.float32(os_).view(np.uint32)
        assert np.array_equal(host_u8(q), oq)


def _state_host(st):
    a = st.cpu().numpy()
    return a[:1].view(np.float32)[0], int(a[1]), int(a[2])


def test_observer_amax_and_max_exact():
    dev = device()
    rng = np.random.default_rng(21)
    st = fp8.new_observer_state(dev)
    ost = oobs.ObserverState()
    for t in range(20):
        n = int(rng.integers(1, 300_000))
        bits = workloads.to_bf16_bits(rng.standard_normal(n).astype(np.float32)
                                      * np.float32(rng.uniform(0.1, 50)))
        fp8.fp8_observe(to_dev_bf16(bits, dev), st, fp8.OBS_MAX)
        oobs.observe(ost, oobs.call_amax(bits), oobs.OBS_MAX)
        m, count, pending = _state_host(st)
        assert m.view(np.uint32) == np.float32(ost.m).view(np.uint32)
        assert count == t + 1 and pending == 0
    s = fp8.fp8_scale_from_state(st)
    assert host_f32(s)[0] == olin.scale_from_amax(ost.m)


def test_observer_nan_propagates():
    dev = device()
    bits = workloads.to_bf16_bits(np.ones(1000, np.float32))
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe(to_dev_bf16(bits, dev), st, fp8.OBS_MAX)
    bits[123] = 0x7FC1
    fp8.fp8_observe(to_dev_bf16(bits, dev), st, fp8.OBS_MAX)
    assert np.isnan(_state_host(st)[0])


@pytest.mark.parametrize("mode", [fp8.OBS_MAX, fp8.OBS_MOVING_AVG])
def test_observer_infinities_and_negative_nan(mode):
    # a call holding -Inf has amax +Inf, which both observers fold to +Inf
    # (m + c * (Inf - m) = Inf); after it a finite call keeps the max at Inf
    # but turns the moving average into NaN (Inf + c * (a - Inf) is
    # Inf - Inf); a NaN pattern with the sign bit set (0xFFC1) counts as NaN.
    # Max: 3, Inf, Inf, NaN; moving average: 3, Inf, NaN, NaN -- each state
    # bit for bit the oracle's, the final scale NaN
    dev = device()
    st = fp8.new_observer_state(dev)
    ost = oobs.ObserverState()
    calls = []
    base = workloads.to_bf16_bits(np.linspace(-3, 2, 5000).astype(np.float32))
    calls.append(base.copy())
    inf_call = base.copy()
    inf_call[77] = 0xFF80                     # -Inf
    calls.append(inf_call)
    calls.append(base.copy())
    nan_call = base.copy()
    nan_call[4000] = 0xFFC1                   # a NaN with the sign bit set
    calls.append(nan_call)
    for c in calls:
        fp8.fp8_observe(to_dev_bf16(c, dev), st, mode, 0.01)
        with np.errstate(invalid="ignore"):     # Inf - Inf in the oracle's update
            oobs.observe(ost, oobs.call_amax(c), mode, 0.01)
        got = _state_host(st)[0]
        want = np.float32(ost.m)
        assert (np.isnan(got) and np.isnan(want)) or got.view(np.uint32) == want.view(np.uint32)
    assert oobs.call_amax(inf_call) == np.inf and np.isnan(oobs.call_amax(nan_call))
    s = host_f32(fp8.fp8_scale_from_state(st))[0]
    assert np.isnan(s) and np.isnan(olin.scale_from_amax(ost.m))


@pytest.mark.parametrize("mode", [fp8.OBS_MAX, fp8.OBS_MOVING_AVG])
def test_two_tower_calibration_und_full(mode):
    # 256 calibration calls of the und tower at full size ([512, 4096] group
    # inputs, [512, 12288] down input), both observers, bit-exact
    dev = device()
    for site in workloads.SITES:
        base = workloads.calib_base("und", site)
        dbase = to_dev_bf16(base, dev).view(-1)
        st = fp8.new_observer_state(dev)
        ost = oobs.ObserverState()
        for t in range(workloads.CALIB_CALLS):
            pos, gain = workloads.calib_spikes("und", site, t, base.size)
            x = workloads.calib_call(base, pos, gain)
            dx = dbase.clone()
            dpos = torch.from_numpy(pos).to(dev)
            dx[dpos] = to_dev_bf16(x.ravel()[pos], dev)
            fp8.fp8_observe(dx, st, mode, 0.01)
            oobs.observe(ost, oobs.call_amax(x), mode, 0.01)
        m, count, _ = _state_host(st)
        assert count == 256
        assert m.view(np.uint32) == np.float32(ost.m).view(np.uint32), site


def test_two_tower_gen_calls_sampled():
    # gen tower, [4096, 12288] down input: a few calls at full size
    dev = device()
    base = workloads.calib_base("gen", "down")
    dbase = to_dev_bf16(base, dev).view(-1)
    for mode in (fp8.OBS_MAX, fp8.OBS_MOVING_AVG):
        st = fp8.new_observer_state(dev)
        ost = oobs.ObserverState()
        for t in range(4):
            pos, gain = workloads.calib_spikes("gen", "down", t, base.size)
            x = workloads.calib_call(base, pos, gain)
            dx = dbase.clone()
            dx[torch.from_numpy(pos).to(dev)] = to_dev_bf16(x.ravel()[pos], dev)
            fp8.fp8_observe(dx, st, mode, 0.01)
            oobs.observe(ost, oobs.call_amax(x), mode, 0.01)
        m = _state_host(st)[0]
        assert m.view(np.uint32) == np.float32(ost.m).view(np.uint32)


def test_moving_average_scales_saturate_forward_inputs():
    # the moving-average scale sits below the per-call maxima of the spiky
    # calls, so quantizing the spikiest call under it must clip; the forward
    # draw is quantized bit-exactly as well
    dev = device()
    base = workloads.calib_base("und", "qkv")
    dbase = to_dev_bf16(base, dev).view(-1)
    st = fp8.new_observer_state(dev)
    best, best_amax = None, -1.0
    for t in range(workloads.CALIB_CALLS):
        pos, gain = workloads.calib_spikes("und", "qkv", t, base.size)
        dx = dbase.clone()
        x = workloads.calib_call(base, pos, gain)
        dx[torch.from_numpy(pos).to(dev)] = to_dev_bf16(x.ravel()[pos], dev)
        fp8.fp8_observe(dx, st, fp8.OBS_MOVING_AVG, 0.01)
        a = float(oobs.call_amax(x))
        if a > best_amax:
            best, best_amax = x, a
    s = fp8.fp8_scale_from_state(st)
    q = host_u8(fp8.fp8_quant_static(to_dev_bf16(best, dev), s))
    assert np.count_nonzero((q & 0x7F) == 0x7E) > 0
    assert np.array_equal(q, olin.quant_static(best, host_f32(s)[0]))
    fwd = workloads.forward_input("und", "qkv")
    qf = host_u8(fp8.fp8_quant_static(to_dev_bf16(fwd, dev), s))
    assert np.array_equal(qf, olin.quant_static(fwd, host_f32(s)[0]))


def test_observe_swiglu_amax():
    dev = device()
    rng = np.random.default_rng(22)
    g = workloads.to_bf16_bits(rng.standard_normal(100_003).astype(np.float32) * 3)
    u = workloads.to_bf16_bits(rng.standard_normal(100_003).astype(np.float32) * 2)
    st = fp8.new_observer_state(dev)
    fp8.fp8_observe_swiglu(to_dev_bf16(g, dev), to_dev_bf16(u, dev), st, fp8.OBS_MAX)
    m = _state_host(st)[0]
    from oracle.swiglu import silu_mul_f64
    ref = np.max(np.abs(silu_mul_f64(g, u)))
    # FP32 evaluation with hardware exp/rcp: a few FP32 ulps
    assert abs(float(m) - ref) <= 8 * 2.0 ** -23 * ref


def test_refusals():
    dev = device()
    x = to_dev_bf16(ALL_BF16[:64], dev)
    with pytest.raises(fp8.Fp8motError) as e:
        fp8.fp8_quant_static(x, None)
    assert e.value.status == 4
    with pytest.raises(ValueError):
        fp8.fp8_quant_static(x.view(8, 8).t(), scalar(1.0, dev))
    # misaligned base pointer: refused, not handled on a slow path
    xb = to_dev_bf16(ALL_BF16[:80], dev)[1:65]
    with pytest.raises(fp8.Fp8motError) as e:
        fp8.fp8_quant_static(xb, scalar(1.0, dev))
    assert e.value.status == 2


@pytest.mark.parametrize("mode", [fp8.OBS_MAX, fp8.OBS_MOVING_AVG])
@pytest.mark.parametrize("n", [1 << 20, 8 << 20])
def test_observer_in_hip_graph_folds_every_replay(mode, n):
    # 1M elements fold in the amax launch itself (last workgroup to arrive),
    # 8M in a second one-thread launch; either way a captured observe folds on
    # every replay and leaves both reduction slots at zero, with eager calls
    # on the same state between replays
    dev = device()
    rng = np.random.default_rng(n + mode)
    draws = [workloads.to_bf16_bits(rng.standard_normal(n).astype(np.float32)
                                    * np.float32(rng.uniform(0.5, 40))) for _ in range(6)]
    st = fp8.new_observer_state(dev)
    ost = oobs.ObserverState()
    x_static = to_dev_bf16(draws[0], dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        warm = fp8.new_observer_state(dev)
        fp8.fp8_observe(x_static, warm, mode)      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8.fp8_observe(x_static, st, mode)
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 0, 0, 0]   # capture ran nothing
    for t, bits in enumerate(draws):
        if t % 2 == 0:
            x_static.copy_(to_dev_bf16(bits, dev))
            g.replay()
        else:
            fp8.fp8_observe(to_dev_bf16(bits, dev), st, mode)
        torch.cuda.synchronize()
        oobs.observe(ost, oobs.call_amax(bits), mode)
        a = st.cpu().numpy()
        assert a[:1].view(np.float32)[0].view(np.uint32) == np.float32(ost.m).view(np.uint32), t
        assert int(a[1]) == t + 1 and int(a[2]) == 0 and int(a[3]) == 0, (t, a.tolist())


@pytest.mark.parametrize("mode", [fp8.OBS_MAX, fp8.OBS_MOVING_AVG])
def test_observer_random_sizes_both_fold_paths(mode):
    # 300 calls on one state with sizes from 1 to 9M elements, so that calls
    # alternate between the in-launch fold (<= 128 workgroups) and the
    # separate fold launch; the state checked against the oracle every call
    dev = device()
    rng = np.random.default_rng(40 + mode)
    pool = workloads.to_bf16_bits(rng.standard_normal(9 << 20).astype(np.float32))
    dpool = to_dev_bf16(pool, dev)
    st = fp8.new_observer_state(dev)
    ost = oobs.ObserverState()
    for t in range(300):
        n = int(rng.integers(1, 9 << 20)) if t % 3 else int(rng.integers(1, 1 << 16))
        off = int(rng.integers(0, (9 << 20) - n + 1)) // 8 * 8
        fp8.fp8_observe(dpool[off:off + n], st, mode)
        oobs.observe(ost, oobs.call_amax(pool[off:off + n]), mode)
        a = st.cpu().numpy()
        assert a[:1].view(np.float32)[0].view(np.uint32) == np.float32(ost.m).view(np.uint32), (t, n)
        assert int(a[1]) == t + 1 and int(a[2]) == 0 and int(a[3]) == 0, (t, n, a.tolist())
