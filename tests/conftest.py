import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "libmoe_oracle.so")):
        oracle.build()
    return oracle


def pytest_sessionfinish(session, exitstatus):
    """With MOE_PARITY_LOG set, write every output comparison of the GPU
    parity tests (bare max|d|/RMS and the rest, tests/gpu_common.py) there as
    JSON lines."""
    path = os.environ.get("MOE_PARITY_LOG")
    if not path:
        return
    mod = sys.modules.get("gpu_common")
    if mod is None:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        for rec in mod.RECORDS:
            f.write(json.dumps(rec) + "\n")
