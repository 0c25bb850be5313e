"""GPU parity: two-input SwiGLU with FP8 output, and the composites
gated_mlp_fp8 / qkv_fp8 (bitwise equal to their parts, one quantization)."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from mlp_fp8_quant_amd import workloads
from oracle import linear as olin
from oracle.formats import e4m3_decode
from oracle.swiglu import silu_mul_f64, silu_mul_fp8

from gpu_util import (check_fp8_tolerance, check_gemm_bf16, check_gemm_f32,
                      device, host_bits, host_f32, host_u8, report, scalar,
                      to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu


def _gu(rng, n, sg=3.0, su=2.0):
    g = workloads.to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(sg))
    u = workloads.to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(su))
    return g, u


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 65537, 2048 * 8192])
def test_swiglu_random(n):
    dev = device()
    rng = np.random.default_rng(n)
    g, u = _gu(rng, n)
    s = np.float32(np.max(np.abs(silu_mul_f64(g, u))) / 448)
    q = fp8.silu_mul_2in_fp8(to_dev_bf16(g, dev), to_dev_bf16(u, dev), scalar(s, dev))
    check_fp8_tolerance(host_u8(q), silu_mul_fp8(g, u, s))


def test_swiglu_rank3_and_saturation():
    dev = device()
    rng = np.random.default_rng(40)
    g, u = _gu(rng, 4 * 96 * 128, 6.0, 4.0)
    s = np.float32(0.01)  # forces saturation of the large products
    dg = to_dev_bf16(g, dev).view(4, 96, 128)
    du = to_dev_bf16(u, dev).view(4, 96, 128)
    q = fp8.silu_mul_2in_fp8(dg, du, scalar(s, dev))
    assert q.shape == (4, 96, 128)
    want = silu_mul_fp8(g, u, s)
    assert np.count_nonzero((want & 0x7F) == 0x7E) > 0
    check_fp8_tolerance(host_u8(q).ravel(), want)


def test_swiglu_special_values():
    dev = device()
    gv = np.array([0.0, -0.0, 0.0, 40.0, 100.0, -1e4, -3e38, 3e38, 17.0, -17.0,
                   np.inf, -np.inf, np.nan, 1.0, -1.0, 0.5], np.float32)
    uv = np.array([2.0, 2.0, -2.0, 0.25, -0.125, 1.0, -1.0, 1.0, 3.0, 3.0,
                   1.0, 1.0, 1.0, 0.0, -0.0, 1e-30], np.float32)
    g, u = workloads.to_bf16_bits(gv), workloads.to_bf16_bits(uv)
    s = np.float32(0.05)
    q = host_u8(fp8.silu_mul_2in_fp8(to_dev_bf16(g, dev), to_dev_bf16(u, dev),
                                     scalar(s, dev)))
    assert np.array_equal(q, silu_mul_fp8(g, u, s))


def test_swiglu_refuses_strided():
    dev = device()
    g = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        fp8.silu_mul_2in_fp8(g.t(), g, scalar(1.0, dev))


def _mlp_setup(wl, dev):
    """Scales and device weights of a gated-MLP workload (oracle-side RTN,
    oracle-side s_h = amax(silu(G) U) / 448 from the oracle's G and U)."""
    x = wl.x
    sx = olin.scale_from_amax(olin.amax_f32(x))
    qx = olin.quant_static(x, sx)
    q = {}
    s = {}
    for k, w in wl.weights.items():
        q[k], s[k] = olin.rtn_weight(w)
    Sg, Ag = olin.gemm_exact(qx, q["gate"])
    Su, Au = olin.gemm_exact(qx, q["up"])
    G = olin.epilogue_bf16(Sg, sx, s["gate"])
    U = olin.epilogue_bf16(Su, sx, s["up"])
    # the down projection's static input scale: amax of the oracle's
    # silu(G)*U over / 448, fixed once and given to both sides
    sh = olin.scale_from_amax(np.float32(np.max(np.abs(silu_mul_f64(G, U)))))
    d = {k: to_dev_u8(v, dev) for k, v in q.items()}
    sc = {k: scalar(v, dev) for k, v in s.items()}
    return dict(x=x, sx=sx, qx=qx, q=q, s=s, G=G, U=U, sh=sh, d=d, sc=sc,
                Sg=Sg, Ag=Ag, Su=Su, Au=Au)


def test_gated_mlp_composite_equals_parts_and_oracle():
    dev = device()
    wl = workloads.gen_tower_mlp()
    c = _mlp_setup(wl, dev)
    dx = to_dev_bf16(c["x"], dev)
    dsx, dsh = scalar(c["sx"], dev), scalar(c["sh"], dev)
    before = fp8.debug_quant_launches()
    y = fp8.gated_mlp_fp8(dx, dsx, c["d"]["gate"], c["sc"]["gate"], c["d"]["up"],
                          c["sc"]["up"], dsh, c["d"]["down"], c["sc"]["down"])
    torch.cuda.synchronize()
    assert fp8.debug_quant_launches() - before == 1   # one shared quantization
    # the five separate calls
    qx = fp8.fp8_quant_static(dx, dsx)
    G = fp8.fp8_linear(qx, c["d"]["gate"], dsx, c["sc"]["gate"])
    U = fp8.fp8_linear(qx, c["d"]["up"], dsx, c["sc"]["up"])
    qh = fp8.silu_mul_2in_fp8(G, U, dsh)
    y2 = fp8.fp8_linear(qh, c["d"]["down"], dsh, c["sc"]["down"])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(fp8.fp8_gate_up_swiglu(qx, c["d"]["gate"], dsx, c["sc"]["gate"],
                                              c["d"]["up"], c["sc"]["up"], dsh), qh)
    # stage-wise against the oracle: qX bit-exact; G and U within 1 BF16 ulp
    # of the oracle's (or, near cancellation, the RNE of an FP32 output
    # within 1e-5 sum|terms|); the SwiGLU codes within one step on <= 0.1%
    assert np.array_equal(host_u8(qx), c["qx"])
    for k, t, S_, A_ in (("gate", G, c["Sg"], c["Ag"]), ("up", U, c["Su"], c["Au"])):
        t32 = host_f32(fp8.fp8_linear(qx, c["d"][k], dsx, c["sc"][k], fp8.OUT_F32))
        n2 = check_gemm_bf16(host_bits(t), t32, S_, A_, olin.epilogue_alpha(c["sx"], c["s"][k]))
        report(f"gen_mlp_{k}_2048x8192x2048_r13_second_clause", n2)
    n_off = check_fp8_tolerance(host_u8(qh).ravel(), silu_mul_fp8(c["G"], c["U"], c["sh"]))
    report("gen_mlp_swiglu_2048x8192_codes_one_step_off_frac", n_off / qh.numel())
    # end to end: the oracle chain, with the tolerance widened by exactly the
    # effect of the SwiGLU codes that differ by one step
    qh_o = silu_mul_fp8(c["G"], c["U"], c["sh"]).reshape(2048, 8192)
    qh_g = host_u8(qh).reshape(2048, 8192)
    S, A = olin.gemm_exact(qh_o, c["q"]["down"])
    alpha = olin.epilogue_alpha(c["sh"], c["s"]["down"])
    dH = np.abs(e4m3_decode(qh_g) - e4m3_decode(qh_o))
    extra = dH @ np.abs(e4m3_decode(c["q"]["down"])).T
    yv = host_bits(y).astype(np.uint32)
    yf = (yv << 16).view(np.float32).astype(np.float64)
    ref = np.float64(alpha) * S
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-300
    bound = np.float64(alpha) * (extra + 1e-5 * A) + ulp
    assert np.all(np.abs(yf - ref) <= bound)


def test_qkv_composite_equals_parts_and_oracle():
    dev = device()
    wl = workloads.split_qkv()
    sx = olin.scale_from_amax(olin.amax_f32(wl.x))
    qx = olin.quant_static(wl.x, sx)
    dx, dsx = to_dev_bf16(wl.x, dev), scalar(sx, dev)
    qs, ss = {}, {}
    for k in ("q", "k", "v"):
        qs[k], ss[k] = olin.rtn_weight(wl.weights[k])
    assert len({float(v) for v in ss.values()}) == 3  # distinct weight scales
    d = {k: to_dev_u8(v, dev) for k, v in qs.items()}
    sc = {k: scalar(v, dev) for k, v in ss.items()}
    before = fp8.debug_quant_launches()
    yq, yk, yv = fp8.qkv_fp8(dx, dsx, d["q"], sc["q"], d["k"], sc["k"], d["v"], sc["v"])
    assert fp8.debug_quant_launches() - before == 1
    for t in (yq, yk, yv):
        assert t.is_contiguous() and t.shape == (3072, 4096)
    dqx = fp8.fp8_quant_static(dx, dsx)
    assert np.array_equal(host_u8(dqx), qx)
    for k, y in zip(("q", "k", "v"), (yq, yk, yv)):
        y2 = fp8.fp8_linear(dqx, d[k], dsx, sc[k])
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        S, A = olin.gemm_exact(qx, qs[k])
        y32 = fp8.fp8_linear(dqx, d[k], dsx, sc[k], fp8.OUT_F32)
        n2 = check_gemm_bf16(host_bits(y), y32.cpu().numpy(), S, A,
                             olin.epilogue_alpha(sx, ss[k]))
        report(f"split_qkv_{k}_3072x4096x4096_r13_second_clause", n2)


def test_split_path_keeps_each_members_codes_not_requantized():
    # Pull request "Description": a fused group re-quantizes each member onto
    # max(s); the split path keeps s_i * qW_i.  With clearly different weight
    # scales (checked first, or the test could not tell the two apart) the
    # GPU output must follow the original codes and differ from the
    # re-quantized ones.
    dev = device()
    rng = np.random.default_rng(42)
    x = workloads.activations(rng, 128, 512)
    ws = [workloads.weights(rng, 256, 512, sd) for sd in (0.02, 0.006, 0.045)]
    sx = olin.scale_from_amax(olin.amax_f32(x))
    qx = olin.quant_static(x, sx)
    qs, ss = zip(*[olin.rtn_weight(w) for w in ws])
    assert len({float(v) for v in ss}) == 3
    rq, smax = olin.requantize_onto_max(qs, ss)
    dqx, dsx = to_dev_u8(qx, dev), scalar(sx, dev)
    for q, sw, r in zip(qs, ss, rq):
        y = fp8.fp8_linear(dqx, to_dev_u8(q, dev), dsx, scalar(sw, dev), fp8.OUT_F32)
        y32 = y.cpu().numpy()
        S, A = olin.gemm_exact(qx, q)
        check_gemm_f32(y32, S, A, olin.epilogue_alpha(sx, sw))
        if sw != smax:
            assert np.count_nonzero(r != q) > 0
            Sr, _ = olin.gemm_exact(qx, r)
            y_req = np.float64(olin.epilogue_alpha(sx, smax)) * Sr
            assert np.count_nonzero(np.abs(y32 - y_req) > 1e-5 * np.float64(
                olin.epilogue_alpha(sx, sw)) * A) > 0


def test_composite_refusals():
    dev = device()
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((64, 64), dtype=torch.uint8, device=dev)
    s = scalar(1.0, dev)
    with pytest.raises(fp8.Fp8motError) as e:
        fp8.qkv_fp8(x, None, w, s, w, s, w, s)
    assert e.value.status == 4
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(fp8.Fp8motError) as e:
        fp8.qkv_fp8(x, s, w, s, w, s, w, s, workspace=small)
    assert e.value.status == 6


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_composites_equal_parts_each_engine(accum):
    # rank-3 input [2, 96, 512]: the composites flatten it to M = 192 rows
    dev = device()
    rng = np.random.default_rng(41)
    x = workloads.activations(rng, 192, 512)
    ws = {k: workloads.weights(rng, *shp, 0.02)
          for k, shp in (("g", (1024, 512)), ("u", (1024, 512)), ("d", (512, 1024)))}
    sx = olin.scale_from_amax(olin.amax_f32(x))
    q, s = {}, {}
    for k, w in ws.items():
        q[k], s[k] = olin.rtn_weight(w)
    d = {k: to_dev_u8(v, dev) for k, v in q.items()}
    sc = {k: scalar(v, dev) for k, v in s.items()}
    dx = to_dev_bf16(x, dev).view(2, 96, 512)
    dsx, dsh = scalar(sx, dev), scalar(0.05, dev)
    y = fp8.gated_mlp_fp8(dx, dsx, d["g"], sc["g"], d["u"], sc["u"], dsh, d["d"],
                          sc["d"], accum=accum)
    assert y.shape == (2, 96, 512)
    qx = fp8.fp8_quant_static(dx, dsx)
    G = fp8.fp8_linear(qx, d["g"], dsx, sc["g"], accum=accum)
    U = fp8.fp8_linear(qx, d["u"], dsx, sc["u"], accum=accum)
    y2 = fp8.fp8_linear(fp8.silu_mul_2in_fp8(G, U, dsh), d["d"], dsh, sc["d"],
                        accum=accum)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    qh = fp8.fp8_gate_up_swiglu(qx, d["g"], dsx, sc["g"], d["u"], sc["u"], dsh,
                                accum=accum)
    assert torch.equal(qh, fp8.silu_mul_2in_fp8(G, U, dsh))
    yq, yk, yv = fp8.qkv_fp8(dx, dsx, d["g"], sc["g"], d["u"], sc["u"], d["g"],
                             sc["g"], accum=accum)
    assert torch.equal(yq.view(torch.int16), G.view(torch.int16))
    assert torch.equal(yk.view(torch.int16), U.view(torch.int16))
    assert torch.equal(yv.view(torch.int16), G.view(torch.int16))


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("M,I,H", [(1, 16, 16), (37, 144, 64), (300, 272, 512),
                                   (513, 1040, 1024)])
def test_gate_up_swiglu_ragged_equals_parts(accum, M, I, H):
    # ragged M, I not a multiple of the 128-column tile, short and long K
    dev = device()
    rng = np.random.default_rng(M + I + H)
    x = workloads.activations(rng, M, H)
    wg = workloads.weights(rng, I, H, 0.02)
    wu = workloads.weights(rng, I, H, 0.02)
    sx = olin.scale_from_amax(olin.amax_f32(x))
    qx = to_dev_u8(olin.quant_static(x, sx), dev)
    (qg, sg), (qu, su) = olin.rtn_weight(wg), olin.rtn_weight(wu)
    dg, du = to_dev_u8(qg, dev), to_dev_u8(qu, dev)
    dsx, dsg, dsu, dsh = (scalar(v, dev) for v in (sx, sg, su, 0.02))
    qh = fp8.fp8_gate_up_swiglu(qx, dg, dsx, dsg, du, dsu, dsh, accum=accum)
    G = fp8.fp8_linear(qx, dg, dsx, dsg, accum=accum)
    U = fp8.fp8_linear(qx, du, dsx, dsu, accum=accum)
    parts = fp8.silu_mul_2in_fp8(G, U, dsh)
    if I >= H:
        # the separate gate and up GEMMs sum along K as the fused kernel does
        assert torch.equal(qh, parts)
    else:
        # H > I with few tiles: fp8_linear sums the even and odd K blocks
        # separately, so G and U may differ in the last FP32 bit and a code
        # may move by a step
        check_fp8_tolerance(host_u8(qh), host_u8(parts))


@pytest.mark.parametrize("ns", [(384, 128, 96), (4096, 1024, 1024), (200, 0, 72)])
@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_qkv_grouped_launch_equals_separate_gemms(ns, accum):
    # qkv_fp8 runs the projections as one grouped launch; with unequal N
    # (GQA-like) and an empty member it still equals three separate
    # fp8_linear calls bit for bit
    dev = device()
    rng = np.random.default_rng(sum(ns) + accum)
    M, H = 300, 512
    x = workloads.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    dx = to_dev_bf16(x.ravel(), dev).view(M, H)
    sx = scalar(0.01, dev)
    ws, ss = [], []
    for n in ns:
        ws.append(to_dev_u8(rng.integers(0, 0x7E, (n, H), dtype=np.uint8), dev))
        ss.append(scalar(0.001 * (1 + len(ss)), dev))
    yq, yk, yv = fp8.qkv_fp8(dx, sx, ws[0], ss[0], ws[1], ss[1], ws[2], ss[2], accum=accum)
    qx = fp8.fp8_quant_static(dx, sx)
    for y, w, s in zip((yq, yk, yv), ws, ss):
        assert y.shape == (M, w.shape[0])
        if w.shape[0]:
            assert torch.equal(y, fp8.fp8_linear(qx, w, sx, s, accum=accum))


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("H", [1040, 1024])
def test_fused_many_tiles_ragged_equals_parts(accum, H):
    # 18 x 33 = 594 fused tiles (more than the GPU holds at once: the exact
    # engine's workgroups walk several, prefetching the next tile's first
    # stages during each epilogue), ragged M and I, K not a multiple of 128
    # (every chunk checked against K) or a multiple of it (whole-stage copies
    # with the stage's column offset as the scalar offset, rows past M and I
    # reading zeros): bitwise the separate gate/up GEMMs + SwiGLU, and the
    # codes of sampled rows (the last ones included) against the oracle
    dev = device()
    M, I = 4357, 4144
    rng = np.random.default_rng(88 + accum + H)
    x = workloads.activations(rng, M, H)
    wg = workloads.weights(rng, I, H, 0.02)
    wu = workloads.weights(rng, I, H, 0.02)
    sx = olin.scale_from_amax(olin.amax_f32(x))
    qx_o = olin.quant_static(x, sx)
    (qg, sg), (qu, su) = olin.rtn_weight(wg), olin.rtn_weight(wu)
    qx = to_dev_u8(qx_o, dev)
    dg, du = to_dev_u8(qg, dev), to_dev_u8(qu, dev)
    sh = np.float32(0.03)
    dsx, dsg, dsu, dsh = (scalar(v, dev) for v in (sx, sg, su, sh))
    qh = fp8.fp8_gate_up_swiglu(qx, dg, dsx, dsg, du, dsu, dsh, accum=accum)
    G = fp8.fp8_linear(qx, dg, dsx, dsg, accum=accum)
    U = fp8.fp8_linear(qx, du, dsx, dsu, accum=accum)
    assert torch.equal(qh, fp8.silu_mul_2in_fp8(G, U, dsh))
    if accum != fp8.ACC_EXACT:
        return
    rows = np.concatenate([np.arange(M - 40, M), np.sort(rng.choice(M - 40, 24, replace=False))])
    Sg, _ = olin.gemm_exact(qx_o[rows], qg)
    Su, _ = olin.gemm_exact(qx_o[rows], qu)
    want = silu_mul_fp8(olin.epilogue_bf16(Sg, sx, sg), olin.epilogue_bf16(Su, sx, su), sh)
    check_fp8_tolerance(host_u8(qh)[rows].ravel(), want)


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_degenerate_composite_shapes(accum):
    # the gated MLP's degenerate shapes, against the oracle chain: no tokens
    # (M = 0), no intermediate channels (I = 0: the weights are empty tensors
    # and y is the down projection of an empty sum) and, for the gate/up
    # half, an empty hidden size (H = 0: G = U = 0, so every SwiGLU code is
    # that of 0); outputs start as NaN bits so a missing write shows
    dev = device()
    M, H, I = 37, 64, 48
    rng = np.random.default_rng(7 + accum)
    x = workloads.activations(rng, M, H)
    dx = to_dev_bf16(x, dev)
    sx, sg, su, sh, sd = (np.float32(v) for v in (0.02, 0.003, 0.004, 0.05, 0.006))
    dsx, dsg, dsu, dsh, dsd = (scalar(v, dev) for v in (sx, sg, su, sh, sd))
    e = lambda *shp: torch.empty(shp, dtype=torch.uint8, device=dev)
    # M = 0
    y0 = fp8.gated_mlp_fp8(dx[:0], dsx, e(I, H).zero_(), dsg, e(I, H).zero_(), dsu, dsh,
                           e(H, I).zero_(), dsd, accum=accum)
    assert y0.shape == (0, H)
    # I = 0: y = epilogue of S = 0 (+0 in BF16)
    qh0 = np.zeros((M, 0), np.uint8)
    want = olin.epilogue_bf16(olin.gemm_exact(qh0, np.zeros((H, 0), np.uint8))[0], sh, sd)
    for run in (fp8.gated_mlp_fp8, fp8.gated_mlp_fp8_noalloc):
        y = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev)
        run(dx, dsx, e(0, H), dsg, e(0, H), dsu, dsh, e(H, 0), dsd, out=y, accum=accum)
        assert np.array_equal(host_bits(y), want)
    # H = 0 for the gate/up half: qh = SwiGLU-FP8 of two zero projections
    qx0 = np.zeros((M, 0), np.uint8)
    G = olin.epilogue_bf16(olin.gemm_exact(qx0, np.zeros((I, 0), np.uint8))[0], sx, sg)
    U = olin.epilogue_bf16(olin.gemm_exact(qx0, np.zeros((I, 0), np.uint8))[0], sx, su)
    want_qh = silu_mul_fp8(G, U, sh).reshape(M, I)
    qh = torch.full((M, I), 0x7F, dtype=torch.uint8, device=dev)
    fp8.fp8_gate_up_swiglu(e(M, 0), e(I, 0), dsx, dsg, e(I, 0), dsu, dsh, out=qh, accum=accum)
    assert np.array_equal(host_u8(qh), want_qh)


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
def test_degenerate_qkv_shapes(accum):
    # qkv_fp8 with an empty hidden size (H = 0: no quantization launch, each
    # projection the epilogue of an empty sum, +0 in BF16) and with no tokens
    dev = device()
    M, ns = 33, (64, 32, 48)
    s = [np.float32(v) for v in (0.02, 0.003, 0.004, 0.005)]
    ds = [scalar(v, dev) for v in s]
    e = lambda *shp: torch.empty(shp, dtype=torch.uint8, device=dev)
    x0 = torch.empty((M, 0), dtype=torch.bfloat16, device=dev)
    outs = tuple(torch.full((M, n), float("nan"), dtype=torch.bfloat16, device=dev) for n in ns)
    before = fp8.debug_quant_launches()
    fp8.qkv_fp8(x0, ds[0], e(ns[0], 0), ds[1], e(ns[1], 0), ds[2], e(ns[2], 0), ds[3],
                outs=outs, accum=accum)
    assert fp8.debug_quant_launches() == before
    for y, n, sw in zip(outs, ns, s[1:]):
        S, _ = olin.gemm_exact(np.zeros((M, 0), np.uint8), np.zeros((n, 0), np.uint8))
        assert np.array_equal(host_bits(y), olin.epilogue_bf16(S, s[0], sw))
    x = to_dev_bf16(workloads.activations(np.random.default_rng(3), 1, 64), dev)[:0]
    yq, yk, yv = fp8.qkv_fp8(x, ds[0], e(ns[0], 64).zero_(), ds[1], e(ns[1], 64).zero_(), ds[2],
                             e(ns[2], 64).zero_(), ds[3], accum=accum)
    assert (yq.shape, yk.shape, yv.shape) == ((0, 64), (0, 32), (0, 48))


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("sh", [1e-5, 1e3])
def test_fused_epilogue_saturates_and_underflows_as_parts(accum, sh):
    # the fused kernel's SwiGLU epilogue at a down-input scale that saturates
    # most codes and at one that takes most to subnormal codes or zero:
    # bitwise the separate gate/up GEMMs + silu_mul_2in_fp8 (I >= H)
    dev = device()
    M, I, H = 300, 1024, 512
    rng = np.random.default_rng(51 + accum)
    x = workloads.activations(rng, M, H)
    wg = workloads.weights(rng, I, H, 0.02)
    wu = workloads.weights(rng, I, H, 0.02)
    sx = olin.scale_from_amax(olin.amax_f32(x))
    qx = to_dev_u8(olin.quant_static(x, sx), dev)
    (qg, sg), (qu, su) = olin.rtn_weight(wg), olin.rtn_weight(wu)
    dg, du = to_dev_u8(qg, dev), to_dev_u8(qu, dev)
    dsx, dsg, dsu, dsh = (scalar(v, dev) for v in (sx, sg, su, sh))
    qh = fp8.fp8_gate_up_swiglu(qx, dg, dsx, dsg, du, dsu, dsh, accum=accum)
    G = fp8.fp8_linear(qx, dg, dsx, dsg, accum=accum)
    U = fp8.fp8_linear(qx, du, dsx, dsu, accum=accum)
    parts = fp8.silu_mul_2in_fp8(G, U, dsh)
    assert torch.equal(qh, parts)
    mag = host_u8(qh) & 0x7F
    if sh < 1:
        assert np.count_nonzero(mag == 0x7E) > mag.size // 2
    else:
        assert np.count_nonzero(mag < 0x08) > mag.size // 2
