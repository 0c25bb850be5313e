"""Seeded synthetic inputs for the static-FP8 Linear workloads.

This module only draws random numbers and rounds them to BF16; it holds none
of the FP8 method's arithmetic (no scales, no quantization, no GEMM).  Both
the HIP path and the CPU oracle take their inputs from here.

Recipe (the pages' own activations -- 256 captured policy-server calls on 32
DROID observations -- and their checkpoints are not available; these draws
stand in for them):

* every draw comes from ``numpy.random.Generator(PCG64(seed))`` with seed 0
  unless stated, in a fixed order per workload: activations, their outlier
  mask, then the weights in the order listed;
* activations are N(0, 1) in float32; "0.5% x20 outliers" multiplies the
  entries selected by a Bernoulli(0.005) mask by 20, in float32, before
  rounding;
* weights are N(0, sigma) in float32 (sigma = 0.02, or 0.015 for the large
  gated MLP);
* everything is rounded to BF16 to nearest-even and returned as uint16 bit
  patterns (numpy arrays, C-contiguous, weights as [out, in]).

Calibration calls for the two-tower layer: site ``j`` has a fixed N(0, 1)
base tensor; call ``t`` multiplies a fresh Bernoulli(0.005) subset of its
entries by a per-call factor drawn from U(5, 30).  The subset is drawn as a
Binomial count followed by uniform positions (with replacement), which is
the same distribution up to rare repeats and needs 0.5% of the draws.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

OUTLIER_P = 0.005
OUTLIER_GAIN = 20.0


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest-even, via torch's CPU cast) -> uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def activations(rng, rows, cols, outliers=True) -> np.ndarray:
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if outliers:
        mask = rng.random((rows, cols), dtype=np.float32) < OUTLIER_P
        x[mask] *= np.float32(OUTLIER_GAIN)
    return to_bf16_bits(x)


def weights(rng, out_f, in_f, std) -> np.ndarray:
    w = rng.standard_normal((out_f, in_f), dtype=np.float32)
    w *= np.float32(std)
    return to_bf16_bits(w)


@dataclass
class Workload:
    name: str
    x: np.ndarray                      # BF16 bits [M, H]
    weights: dict = field(default_factory=dict)  # name -> BF16 bits [out, in]


def single_linear(seed=0, M=64, K=512, N=512) -> Workload:
    """One static FP8 Linear: X [64, 512] with outliers, W [512, 512]."""
    rng = _rng(seed)
    x = activations(rng, M, K, outliers=True)
    w = weights(rng, N, K, 0.02)
    return Workload("single_linear_64x512x512", x, {"w": w})


def gated_mlp(seed=0, M=2048, H=2048, I=8192, std=0.02, name=None) -> Workload:
    """Gated MLP with split gate/up: X [M, H]; Wg, Wu [I, H]; Wd [H, I]."""
    rng = _rng(seed)
    x = activations(rng, M, H, outliers=True)
    wg = weights(rng, I, H, std)
    wu = weights(rng, I, H, std)
    wd = weights(rng, H, I, std)
    name = name or f"gated_mlp_M{M}_H{H}_I{I}"
    return Workload(name, x, {"gate": wg, "up": wu, "down": wd})


def gen_tower_mlp(seed=0) -> Workload:
    """Gen-tower gated MLP: M=2048 tokens, H=2048, I=8192."""
    return gated_mlp(seed, 2048, 2048, 8192, 0.02, "gen_mlp_M2048_H2048_I8192")


def super_mlp(seed=0) -> Workload:
    """Large gated MLP: M=16384, H=5120, I=25600, weights N(0, 0.015)."""
    return gated_mlp(seed, 16384, 5120, 25600, 0.015,
                     "super_mlp_M16384_H5120_I25600")


def split_qkv(seed=0, M=3072, H=4096, N=4096) -> Workload:
    """Split Q/K/V: X [2 x 1536, 4096] (no outliers); Wq, Wk, Wv [4096, 4096]."""
    rng = _rng(seed)
    x = activations(rng, M, H, outliers=False)
    ws = {k: weights(rng, N, H, 0.02) for k in ("q", "k", "v")}
    return Workload(f"split_qkv_M{M}_H{H}_N{N}", x, ws)


# ---------------------------------------------------------------------------
# Two-tower decoder layer (und M=512, gen M=4096; H=4096, I=12288)
# ---------------------------------------------------------------------------

LAYER_H = 4096
LAYER_I = 12288
TOWER_M = {"und": 512, "gen": 4096}
# Linear inputs of one tower: the group input of q/k/v, of o, of gate/up and
# the input of down.  Each is one observer site.
SITES = ("qkv", "o", "gateup", "down")
SITE_COLS = {"qkv": LAYER_H, "o": LAYER_H, "gateup": LAYER_H, "down": LAYER_I}
PROJ_SHAPES = {  # [out, in]
    "q": (LAYER_H, LAYER_H), "k": (LAYER_H, LAYER_H), "v": (LAYER_H, LAYER_H),
    "o": (LAYER_H, LAYER_H), "gate": (LAYER_I, LAYER_H), "up": (LAYER_I, LAYER_H),
    "down": (LAYER_H, LAYER_I),
}
CALIB_CALLS = 256


def layer_weights(tower, seed=0) -> dict:
    """The 7 projection weights of one tower, N(0, 0.02), BF16 bits."""
    rng = _rng((seed, 1 if tower == "und" else 2))
    return {p: weights(rng, *PROJ_SHAPES[p], 0.02) for p in PROJ_SHAPES}


def calib_base(tower, site, seed=0, rows=None) -> np.ndarray:
    """Fixed N(0,1) base tensor of one observer site (BF16 bits)."""
    rng = _rng((seed, 10 + list(TOWER_M).index(tower), SITES.index(site)))
    m = TOWER_M[tower] if rows is None else rows
    return activations(rng, m, SITE_COLS[site], outliers=False)


def calib_spikes(tower, site, t, n, seed=0):
    """Spike positions (flat indices into n elements) and factor of call t."""
    rng = _rng((seed, 100 + list(TOWER_M).index(tower), SITES.index(site), t))
    gain = np.float32(rng.uniform(5.0, 30.0))
    count = rng.binomial(n, OUTLIER_P)
    pos = rng.integers(0, n, size=count, dtype=np.int64)
    return pos, gain


def calib_call(base_bits, pos, gain) -> np.ndarray:
    """Materialize one calibration call: base with spikes multiplied by gain."""
    x = (base_bits.astype(np.uint32) << np.uint32(16)).view(np.float32).ravel().copy()
    x[pos] = x[pos] * gain
    return to_bf16_bits(x).reshape(base_bits.shape)


def calib_spike_values(base_bits, pos, gain) -> np.ndarray:
    """The BF16 bits of one call at its spike positions only: what
    calib_call(base_bits, pos, gain).ravel()[pos] holds (every other entry of
    the call equals the base)."""
    x = (base_bits.ravel()[pos].astype(np.uint32) << np.uint32(16)).view(np.float32)
    return to_bf16_bits(x * gain)


def forward_input(tower, site, seed=0) -> np.ndarray:
    """Forward-pass input of one site: one further draw of the calibration
    distribution (base tensor of its own, spikes at a fresh per-call gain)."""
    m = TOWER_M[tower]
    rng = _rng((seed, 1000 + list(TOWER_M).index(tower), SITES.index(site)))
    x = rng.standard_normal((m, SITE_COLS[site]), dtype=np.float32)
    gain = np.float32(rng.uniform(5.0, 30.0))
    mask = rng.random(x.shape, dtype=np.float32) < OUTLIER_P
    x[mask] *= gain
    return to_bf16_bits(x)


# Configurations by name (parity cases and the bench workload).
CONFIGS = {
    "single_linear": single_linear,
    "gen_mlp": gen_tower_mlp,
    "split_qkv": split_qkv,
    "super_mlp": super_mlp,
}
