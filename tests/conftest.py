import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """libbsattn loaded through the binding (built first if nothing is built)."""
    from head_masked_attention_amd import build as _build
    import head_masked_attention_amd as hm
    if not os.path.exists(hm.LIB_PATH):
        _build.build()
    return hm.load_library()


@pytest.fixture(scope="session")
def cuda():
    if not gpu_available():
        pytest.fail("a GPU test ran without a visible GPU")
    import torch
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    """Name every GPU test on the real stderr before it touches the GPU."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"[gpu-test] start {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
