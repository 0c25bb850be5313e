"""GPU check of the MFMA-ceiling measurement aid the benchmark times beside
the GEMM kernels (not a step of the path): the FLOP count it reports is the
work it issues -- 8 MFMAs per iteration per wave, 8 waves per workgroup, one
workgroup per CU -- so its measured rate must stay below the published dense
peak of the instruction it runs (a dropped or double-counted MFMA would
break that), and the sink is never written for finite data."""

import numpy as np
import pytest
import torch

import mlp_fp8_quant_amd as fp8

from gpu_util import device

pytestmark = pytest.mark.gpu

PEAK_TFLOPS = {fp8.ACC_EXACT: 2500.0, fp8.ACC_FP8_MFMA: 5000.0}
K_PER_MFMA = {fp8.ACC_EXACT: 16, fp8.ACC_FP8_MFMA: 64}


def _codes(n, seed, dev):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, n, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes: 1.0 instead
    return torch.from_numpy(c).to(dev)


@pytest.mark.parametrize("accum", [fp8.ACC_EXACT, fp8.ACC_FP8_MFMA])
@pytest.mark.parametrize("na,nb", [(64, 64), (4099, 1 << 20)])
def test_mfma_ceiling_flops_and_rate(accum, na, nb):
    dev = device()
    a, b = _codes(na, na, dev), _codes(nb, nb + 1, dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4000
    flops = fp8.mfma_ceiling(a, b, iters, sink, accum)
    assert flops == cus * 8 * 8 * iters * 2.0 * 32 * 32 * K_PER_MFMA[accum]
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        fp8.mfma_ceiling(a, b, iters, sink, accum)
    e1.record()
    torch.cuda.synchronize()
    tflops = 5 * flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"mfma ceiling accum={accum} na={na} nb={nb}: {tflops:.0f} TFLOP/s", flush=True)
    assert 0.05 * PEAK_TFLOPS[accum] < tflops <= 1.02 * PEAK_TFLOPS[accum]
    assert float(sink.item()) == 0.0
