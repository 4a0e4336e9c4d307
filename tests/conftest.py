import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Other compiled copies of the oracle and of the C ABI's host layer (the
# sanitizer builds made by test_sanitizers_cpu.py) replace the default ones
# when these name them.
if os.environ.get("TL_TEST_ORACLE_LIB"):
    from oracle import oracle as _O
    _O._override.append(_O._bind(os.environ["TL_TEST_ORACLE_LIB"]))
if os.environ.get("TL_TEST_LORA_LIB"):
    from tenant_lora_serving_amd import lora as _B
    _B.LIB_PATH = os.environ["TL_TEST_LORA_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs; still CPU-only")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is present; on a CPU-only host they are
    # reported as skipped rather than failing at import.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
