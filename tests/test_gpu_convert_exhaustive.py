"""GPU check, over every FP32 bit pattern, of the conversions the path's
kernels use (model card "Cosmos3-Nano-Policy-DROID, FP8 + RTN ...", "Scheme":
E4M3 round to nearest even; the library saturates to +-448, maps NaN to 0x7F
and keeps the sign of zero; BF16 round to nearest even), through the
fp8mot_convert_f32 verification aid, which runs the kernels' own helpers:
the packed E4M3 conversion (quantize and SwiGLU bodies, the GEMMs' FP8
output), the integer E4M3 encoder (the elementwise tails) and the packed BF16
conversion (the GEMM epilogues).

Running the oracle on all 2^32 inputs would take minutes of CPU, so the
sweep proves equality with it another way.  Over the non-negative patterns
u = 0 .. 0x7F800000 (+0 up to +Inf) the FP32 value grows with u, and the
oracle's code (a nearest-value search over the sorted magnitudes, then a
saturation) never decreases with it.  The test checks on the GPU that the
kernel's output never decreases there either, and collects every u where it
changes; the oracle is then evaluated at both sides of each change and at the
two ends.  Two non-decreasing functions that agree at both ends of every run
where one of them is constant agree everywhere.  The negative patterns must
give the positive pattern's result with the sign bit set, and every NaN
pattern (either sign, any payload) 0x7F for E4M3 and a BF16 NaN for BF16.
"""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8
from oracle.formats import e4m3_encode, f32_to_bf16

from gpu_util import device

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28                 # patterns per launch
POS_INF = 0x7F800000            # the last pattern of the ordered range
INT32_MIN = -(1 << 31)

KINDS = {
    "e4m3_packed": (fp8.CONV_E4M3_PACKED, 0x80, 126),
    "e4m3_int": (fp8.CONV_E4M3_INT, 0x80, 126),
    # every BF16 pattern from +0 to +Inf is the rounding of its own FP32
    # extension, so the output takes all 0x7F81 of them: 0x7F80 changes
    "bf16": (fp8.CONV_BF16, 0x8000, 0x7F80),
}


def _as_int(t, kind):
    if kind == fp8.CONV_BF16:
        return t.view(torch.int16).to(torch.int32) & 0xFFFF
    return t.to(torch.int32)


def _oracle(u, kind):
    x = np.asarray(u, np.uint32).view(np.float32)
    if kind == fp8.CONV_BF16:
        return f32_to_bf16(x).astype(np.int64)
    return e4m3_encode(x).astype(np.int64)


@pytest.mark.parametrize("name", list(KINDS))
def test_conversion_on_every_fp32_pattern(name):
    kind, sign_bit, n_changes = KINDS[name]
    dev = device()
    seen_u, seen_v = [], []       # (pattern, kernel output) at both sides of each change
    prev = None                   # kernel output at the pattern before the chunk
    for c in range((1 << 31) // CHUNK):
        start = c * CHUNK
        print(f"{name}: patterns {start:#010x}.. and their negatives", flush=True)
        u = torch.arange(start, start + CHUNK, dtype=torch.int64, device=dev).to(torch.int32)
        v = _as_int(fp8.convert_f32(u.view(torch.float32), kind), kind)
        w = _as_int(fp8.convert_f32(torch.bitwise_or(u, INT32_MIN).view(torch.float32), kind), kind)
        nf = max(0, min(CHUNK, POS_INF + 1 - start))       # ordered patterns in this chunk
        if nf < CHUNK:                                       # NaN patterns, both signs
            if kind == fp8.CONV_BF16:
                assert bool(((v[nf:] & 0x7FFF) > 0x7F80).all()), "BF16 NaN lost"
                assert bool(((w[nf:] & 0x7FFF) > 0x7F80).all()), "BF16 NaN lost"
            else:
                assert bool((v[nf:] == 0x7F).all()) and bool((w[nf:] == 0x7F).all())
        if nf == 0:
            continue
        vf = v[:nf]
        assert torch.equal(w[:nf], vf | sign_bit), "negative pattern is not the sign-flipped positive"
        seq, base = (vf, start) if prev is None else (torch.cat([prev, vf]), start - 1)
        d = seq[1:] - seq[:-1]
        assert bool((d >= 0).all()), "output decreases somewhere"
        j = torch.nonzero(d).flatten()
        seen_u += [base + j.cpu().numpy(), base + 1 + j.cpu().numpy()]
        seen_v += [seq[j].cpu().numpy(), seq[j + 1].cpu().numpy()]
        if prev is None:
            seen_u.append(np.array([start]))
            seen_v.append(vf[:1].cpu().numpy())
        prev = vf[-1:]
    seen_u.append(np.array([POS_INF]))
    seen_v.append(prev.cpu().numpy())
    U = np.concatenate(seen_u).astype(np.int64)
    V = np.concatenate(seen_v).astype(np.int64)
    assert (len(U) - 2) // 2 == n_changes
    want = _oracle(U, kind)
    bad = np.flatnonzero(V != want)
    assert bad.size == 0, [(hex(int(U[i])), hex(int(V[i])), hex(int(want[i]))) for i in bad[:8]]


@pytest.mark.parametrize("n", [4, 12, 1000, 4096 + 8, 3 * 65536 + 4])
def test_conversion_of_short_inputs_against_oracle(n):
    """Short and ragged lengths (fewer groups than one workgroup, a
    partial last workgroup, several grid strides' worth) on random patterns
    of every class: the kernels' result for each element is the oracle's."""
    dev = device()
    print(f"convert n={n}", flush=True)
    rng = np.random.default_rng(n)
    bits = rng.integers(0, 1 << 32, n, dtype=np.int64).astype(np.uint32)
    bits[: min(n, 8)] = [0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0xFF800001,
                         0x43E00000, 0x3A800000][: min(n, 8)]
    x = torch.from_numpy(bits.view(np.float32).copy()).to(dev)
    for kind in (fp8.CONV_E4M3_PACKED, fp8.CONV_E4M3_INT):
        got = fp8.convert_f32(x, kind).cpu().numpy()
        assert np.array_equal(got, e4m3_encode(bits.view(np.float32)))
    got = fp8.convert_f32(x, fp8.CONV_BF16).view(torch.int16).cpu().numpy().view(np.uint16)
    want = f32_to_bf16(bits.view(np.float32))
    nan = np.isnan(bits.view(np.float32))
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)
