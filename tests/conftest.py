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


@pytest.fixture(params=["fused", "separate"])
def kernel_choice(request):
    """Runs a GPU test once with the selection fused into the product (the
    default of spax_layer_step) and once with the stand-alone selection
    kernel followed by the list-reading product."""
    import activation_sparse_decode_token_amd as spax
    spax.set_kernel_choice({"fused": spax.KERNEL_AUTO,
                            "separate": spax.KERNEL_SEPARATE}[request.param])
    yield request.param
    spax.set_kernel_choice(spax.KERNEL_AUTO)
