import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running full-size case")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


# spax_layer.kernel values (SPAX_KERNEL_*), by test id
KERNELS = {"layer": 0, "separate": 1, "per_group": 2}


@pytest.fixture(params=["layer", "per_group", "separate"])
def kernel_choice(request):
    """Runs a GPU test once per launch form of spax_layer_step: the one-launch
    layer kernel (the default), one fused rank + product launch per group,
    and the stand-alone selection kernel followed by the list-reading
    product. Returns the spax_layer.kernel value."""
    return KERNELS[request.param]
