import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-only checks, opt in with MLA_SLOW=1")
    # Oracle worker processes fork from a server started here, before any test touches the
    # GPU, so no process with an initialised GPU runtime ever forks or execs.
    import multiprocessing as mp
    import multiprocessing.forkserver as fs
    mp.set_forkserver_preload(["numpy", "oracle", "synthetic", "tests.oracle_side"])
    fs.ensure_running()


def pytest_collection_modifyitems(config, items):
    if os.environ.get("MLA_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow check; set MLA_SLOW=1 to run")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def nl1(got, ref):
    """Normalised L1 error sum|got-ref| / sum|ref| ("mean relative error")."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).sum() / np.abs(ref).sum())
