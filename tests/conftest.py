import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")

    # A GPU test never passes by skipping: on a host without a GPU the
    # gpu-marked tests are deselected with -m "not gpu"; run with -m gpu they
    # fail loudly when no device is present (gpu_util.device()).
