"""The C ABI from plain C: tests/c_abi_driver (built by __graft_entry__.build())
allocates with hipMalloc, creates its own stream, sizes the workspace with
lrs_scan_workspace_bytes, checks that bad arguments and a missing workspace
are rejected, and runs lrs_scan_fwd + lrs_scan_bwd; its outputs must match the
fp64 oracle to the fp32 bar.  One shape fits a workgroup per channel, the other
spans several look-back chunks (and so needs the workspace)."""
import os
import subprocess

import numpy as np
import pytest

from linear_recurrence_scan_diagonal_amd import inputs as I
from gpu_util import log
from test_gpu_scan import compare, oracle_scan

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi_driver")


@pytest.mark.parametrize("B,D,T", [(2, 3, 1000), (1, 3, 20000)])
def test_c_driver_matches_oracle(tmp_path, B, D, T):
    assert os.path.exists(DRIVER), "tests/c_abi_driver is not built; run __graft_entry__.build()"
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=15000 + T)
    x = I.scan_inputs(w)
    C = B * D
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for k in ("a", "b", "g"):
            f.write(np.ascontiguousarray(x[k], dtype=np.float32).tobytes())
        f.write(np.ascontiguousarray(x["h0"], dtype=np.float32).tobytes())
    log(f"c_abi_driver {B} {D} {T}")
    res = subprocess.run([DRIVER, str(B), str(D), str(T), str(src), str(dst)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = np.fromfile(dst, dtype=np.float32)
    assert out.size == 3 * C * T + C
    n = C * T
    got = {"h": out[:n].reshape(C, T), "da": out[n:2 * n].reshape(C, T),
           "db": out[2 * n:3 * n].reshape(C, T), "dh0": out[3 * n:]}
    compare(got, oracle_scan(x), tag=f"c driver {B}x{D}x{T}")
