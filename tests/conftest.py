import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def relerr(x, ref) -> float:
    """max |x - ref| / (1 + |ref|): the parity metric used for every output tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise AssertionError(f"shape mismatch {x.shape} vs {ref.shape}")
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref) / (1.0 + np.abs(ref))))


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture
def plan():
    """plan(**fields): from here to the end of the test, library calls made
    without explicit options pass these lrs_options fields (see
    binding.plan_options); later calls override earlier fields."""
    import contextlib
    import linear_recurrence_scan_diagonal_amd as lrs
    with contextlib.ExitStack() as stack:
        def set_fields(**fields):
            stack.enter_context(lrs.plan_options(**fields))
        yield set_fields
