"""GPU check of the read/write ceiling kernel the benchmark times beside the
quantize and SwiGLU kernels (a measurement aid, not a step of the path):
out[i] is the low byte of a[i], or of a[i] ^ b[i], over ragged lengths that
exercise the 16-element units and the one-by-one tail."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8

from gpu_util import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 65537, 3_000_001])
@pytest.mark.parametrize("two", [False, True])
def test_rw_ceiling_bytes(n, two):
    dev = device()
    rng = np.random.default_rng(n + two)
    a = rng.integers(0, 65536, n, dtype=np.int64).astype(np.uint16)
    b = rng.integers(0, 65536, n, dtype=np.int64).astype(np.uint16)
    da = torch.from_numpy(a.view(np.int16)).to(dev)
    db = torch.from_numpy(b.view(np.int16)).to(dev) if two else None
    out = torch.empty(n, dtype=torch.uint8, device=dev)
    fp8.rw_ceiling(da, db, out)
    want = ((a ^ b) if two else a) & 0xFF
    assert np.array_equal(out.cpu().numpy(), want.astype(np.uint8))
