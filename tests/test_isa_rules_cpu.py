"""The device code obeys two rules of the target machines, checked on the
assembly hipcc emits for every kernel of the library (CPU only, no GPU):

* no writes through the scalar data cache: no scalar memory stores or
  atomics, no write-back or discard of that cache (every store goes through
  the vector memory path);
* no packed FP32 arithmetic (the library is compiled without it).
"""

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from mlp_fp8_quant_amd import build as b

HIPCC = b.HIPCC
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")

SCALAR_WRITE = re.compile(r"^\s*s_(store|atomic|buffer_store|buffer_atomic|scratch_store|dcache_wb|dcache_discard)")
PACKED_F32 = re.compile(r"^\s*v_pk_(add|mul|fma|mov)_f32")


@pytest.fixture(scope="module")
def assembly():
    out = tempfile.mkdtemp(prefix="fp8mot_isa_")

    def emit(src):
        path = os.path.join(out, src.replace(".hip", ".s"))
        subprocess.run([HIPCC, *b.FLAGS, "--cuda-device-only", "-S",
                        os.path.join(b.CSRC, src), "-o", path],
                       check=True, capture_output=True, text=True)
        return src, open(path).read().splitlines()

    try:
        with ThreadPoolExecutor(max_workers=3) as ex:
            yield dict(ex.map(emit, b.SOURCES))
    finally:
        shutil.rmtree(out, ignore_errors=True)


def test_every_source_has_kernels(assembly):
    for src in ("elementwise.hip", "gemm.hip"):
        assert any(re.match(r"^_Z\S*:", l) for l in assembly[src]), src


def test_no_scalar_cache_writes(assembly):
    bad = [(src, l.strip()) for src, lines in assembly.items() for l in lines if SCALAR_WRITE.match(l)]
    assert not bad, bad[:10]


def test_no_packed_fp32(assembly):
    bad = [(src, l.strip()) for src, lines in assembly.items() for l in lines if PACKED_F32.match(l)]
    assert not bad, bad[:10]


def test_vector_stores_and_mfma_present(assembly):
    # the checks above are only meaningful on real kernel code
    gemm = assembly["gemm.hip"]
    assert any(re.match(r"^\s*v_mfma_", l) for l in gemm)
    assert any(re.match(r"^\s*buffer_store_", l) for l in gemm)


def _kernels(lines):
    """Kernel name -> its assembly lines (from its label to .Lfunc_end)."""
    out, name = {}, None
    for l in lines:
        m = re.match(r"^(_Z\S*):", l)
        if m:
            name = m.group(1)
            out[name] = []
        elif name is not None:
            if l.startswith(".Lfunc_end"):
                name = None
            else:
                out[name].append(l)
    return out


@pytest.mark.parametrize("engine,mnemonic", [(0, "v_mfma_f32_32x32x16_f16"),
                                             (1, "v_mfma_f32_32x32x64_f8f6f4")])
def test_mfma_ceiling_loop_keeps_its_mfmas(assembly, engine, mnemonic):
    """The measurement loop of fp8mot_mfma_ceiling issues its eight MFMAs per
    iteration inside one backward branch, and nothing spills: the compiler
    dropped none of the work the benchmark counts."""
    ks = {k: v for k, v in _kernels(assembly["mfma_ceiling.hip"]).items()
          if "mfma_ceiling_kernel" in k and f"ILi{engine}E" in k}
    assert len(ks) == 1, list(ks)
    body = next(iter(ks.values()))
    assert not any("scratch_" in l for l in body)
    found = False
    for i, l in enumerate(body):
        m = re.match(r"^(\.LBB\w+):", l)
        if not m:
            continue
        for j in range(i + 1, len(body)):
            if re.match(rf"^\s*s_cbranch_\w+\s+{re.escape(m.group(1))}\b", body[j]):
                n = sum(1 for x in body[i:j] if x.strip().startswith(mnemonic))
                found |= n == 8
                break
    assert found


@pytest.mark.parametrize("kind,mnemonic", [(0, "v_cvt_pk_fp8_f32"), (2, "v_cvt_pk_bf16_f32")])
def test_conversion_aid_runs_the_instructions_the_kernels_use(assembly, kind, mnemonic):
    """fp8mot_convert_f32 checks the kernels' conversions over all FP32
    inputs; that holds for the kernels only if its kernel issues the same
    conversion instruction they do, and the kernels issue it too."""
    ks = {k: v for k, v in _kernels(assembly["verify.hip"]).items()
          if "convert_f32_kernel" in k and f"ILi{kind}E" in k}
    assert len(ks) == 1, list(ks)
    assert any(l.strip().startswith(mnemonic) for l in next(iter(ks.values())))
    users = ("elementwise.hip", "gemm.hip") if kind == 0 else ("gemm.hip",)
    for src in users:
        assert any(l.strip().startswith(mnemonic) for l in assembly[src]), src
