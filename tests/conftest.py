import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))
if str(Path(__file__).resolve().parent) not in sys.path:
    sys.path.insert(0, str(Path(__file__).resolve().parent))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def built_lib():
    """Path of libpaged_gqa.so, building it first if this tree has none yet."""
    from paged_gqa_kv_02_amd import build as B
    if not B.LIB.exists():
        B.build()
    return B.LIB
