import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The sanitizer test runs the host checks against a sanitizer build of the C ABI.
    lib = os.environ.get("MOE_TEST_PERMUTE_LIB")
    if lib:
        from mixture_experts_token_amd import binding

        binding.LIB_PATH = lib
        binding._lib = None


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def hip_device():
    """cuda:0 with the HIP library loaded; a GPU test fails loudly if either is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from mixture_experts_token_amd import binding

    binding.load_library()  # raises if the HIP extension was not built
    return torch.device("cuda:0")
