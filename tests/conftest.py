import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running case (still part of the default run)")


def read_golden(name):
    """Rows of whitespace-separated fields from tests/golden/<name>, comments stripped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(params=[1, 2, 3], ids=["rowstream", "tiled", "splitk"])
def schedule(request):
    """Run a GPU test with each GEMM kernel forced (row-streaming = 1, tiled = 2, split-k = 3 for
    single-expert calls with g <= 16, other calls as automatic): all must meet the same contract."""
    import block_scaled_fp4_quant_amd as fp4
    assert request.param in (fp4.SCHEDULE_ROWSTREAM, fp4.SCHEDULE_TILED, fp4.SCHEDULE_SPLITK)
    fp4.set_gemm_schedule(request.param)
    yield request.param
    fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
