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
