"""CPU oracle for the static per-tensor FP8 (E4M3) W8A8 Linear stack.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library and imports
nothing from ``mlp_fp8_quant_amd``.

The oracle is plain and slow on purpose: NumPy in float64 (or float32 where a
step is specified as a single float32 rounding), with every function citing
the passage of the source pages it follows.  The pages are

* "Cosmos3-Nano-Policy-DROID, FP8 + RTN + moving-average activation observer"
  (a Hugging Face model card; sections "Scheme", "Verification",
  "Fake quant" setup), and
* "Load static FP8 Cosmos3 Nano/Super checkpoints without re-quantizing them"
  (TensorRT-LLM pull request 17476; sections "Description", "What changed",
  "Test Coverage" and the commit messages).

Modules
-------
formats   E4M3 (OCP E4M3FN) decode/encode and BF16 rounding.
linear    static activation quantization, RTN weight quantization, the exact
          FP8 GEMM and its epilogues, and the fused-group re-quantization
          failure mode.
swiglu    two-input SiLU(G)*U with direct FP8 emission; the alpha (gain inside
          the sigmoid) / beta (offset on up) variant and the one-input form
          with gate and up adjacent in one tensor.
observer  per-call amax and the max / moving-average observers.
rowwise   per-row FP8: per-channel weight and per-token activation scales.

Every function here is pinned by a ``-m "not gpu"`` test in ``tests/`` to
something other than itself (closed forms, library conversions, exact integer
arithmetic, brute force).  A function without such a pin would be listed here
as "parity unpinned"; at present there is none.
"""

from . import formats, linear, observer, rowwise, swiglu  # noqa: F401
