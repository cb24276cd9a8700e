import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sparse_gradient_reduction_amd as sg
    sg.lib()  # raises if the HIP library is missing: no fallback exists
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def rocrand_probe():
    """A small host program that prints rocRAND's Philox-4x32-10 block for
    each "c0 c1 c2 c3 k0 k1" line of its input (test-only reference)."""
    import shutil
    import subprocess
    import tempfile
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND probe")
    d = tempfile.mkdtemp(prefix="philox_probe_")
    exe = os.path.join(d, "probe")
    subprocess.check_call([hipcc, "-O1", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           os.path.join(ROOT, "tests", "rocrand_philox_probe.cpp"), "-o", exe])
    yield exe
    shutil.rmtree(d, ignore_errors=True)
