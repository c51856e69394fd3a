import os
import sys

# torch first, so that libpuro binds to the HIP runtime torch loaded (one runtime per process).
import torch  # noqa: F401
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP GPU (MI355X); runs the libpuro kernels")


def gpu_available() -> bool:
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.lib()
    return o


@pytest.fixture(scope="session")
def puro():
    if not gpu_available():
        pytest.skip("no HIP device")
    import blockwise_fp8_gemm_x128_amd as p
    from blockwise_fp8_gemm_x128_amd import binding
    binding.lib()
    return binding
