"""Short channels on the GPU: the sequential per-channel kernels (one lane per
channel) and the packed kernels (whole channels per workgroup, resets at
channel starts), chosen below the measured crossovers, against the fp64
oracle, to the fp32 bar 1e-5, on the [B,D,T] layout: every T around the
crossovers and the 16-byte/element-wise paths (T divisible by 4 or not,
channels straddling rows and waves, partial last blocks), grad_b written over
grad_h, each kernel family forced at the same T through the overrides, and
bit-exact integer inputs."""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from gpu_util import DEV, from_dev, log, to_dev
from test_gpu_scan import compare, oracle_scan, run_scan

pytestmark = pytest.mark.gpu

SHORT = [1, 2, 3, 4, 5, 7, 8, 12, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 255, 257]


@pytest.mark.parametrize("T", SHORT)
@pytest.mark.parametrize("B,D", [(1, 1), (3, 100), (2, 700)])
def test_short_channels(B, D, T):
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9500 + B * 31 + D + T * 7)
    x = I.scan_inputs(w)
    compare(run_scan(x, B, D, T, "bdt"), oracle_scan(x), tag=f"short/{B}x{D}x{T}")


@pytest.mark.parametrize("mode", ["serial", "packed", "parallel"])
@pytest.mark.parametrize("T", [3, 6, 16, 40, 300, 1000, 2047, 4096])
def test_forced_kernel(plan, mode, T):
    """Each kernel family at any T through the plan options serial_fwd_max_t,
    serial_bwd_max_t and packed_max_t (packed falls back to one channel per
    workgroup where no channel fits a packed block)."""
    big = 1 << 40
    ser = big if mode == "serial" else 0
    plan(serial_fwd_max_t=ser, serial_bwd_max_t=ser, packed_max_t=big if mode == "packed" else 0)
    B, D = 2, 333
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9600 + T)
    x = I.scan_inputs(w)
    compare(run_scan(x, B, D, T, "bdt"), oracle_scan(x), tag=f"forced-{mode}/{T}")


@pytest.mark.parametrize("T", [13, 32])
def test_short_backward_in_place(T):
    B, D = 4, 77
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9700 + T)
    x = I.scan_inputs(w)
    a, b, g = (to_dev(x[k], B, D, T, "bdt") for k in ("a", "b", "g"))
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    h = lrs.scan_fwd(a, b, h0)
    da, db, dh0 = lrs.scan_bwd(a, h, g, h0, grad_b=g)
    torch.cuda.synchronize()
    assert db.data_ptr() == g.data_ptr()
    got = {"h": from_dev(h, B, D, T, "bdt"), "da": from_dev(da, B, D, T, "bdt"),
           "db": from_dev(db, B, D, T, "bdt"), "dh0": dh0.cpu().numpy().reshape(-1)}
    compare(got, oracle_scan(x), tag=f"short-in-place/{T}")


def test_short_fused_call():
    """lrs_scan_fwd_bwd with short channels: the sequential pair (h wanted) and
    the one-kernel form (h left out) agree with the oracle."""
    B, D, T = 3, 257, 24
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9800)
    x = I.scan_inputs(w)
    a, b, g = (to_dev(x[k], B, D, T, "bdt") for k in ("a", "b", "g"))
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    ref = oracle_scan(x)
    for want_h in (True, False):
        h, da, db, dh0 = lrs.scan_fwd_bwd(a, b, g, h0, want_h=want_h)
        torch.cuda.synchronize()
        got = {"da": from_dev(da, B, D, T, "bdt"), "db": from_dev(db, B, D, T, "bdt"),
               "dh0": dh0.cpu().numpy().reshape(-1)}
        if want_h:
            got["h"] = from_dev(h, B, D, T, "bdt")
        compare(got, {k: ref[k] for k in got}, tag=f"short-fused/h={want_h}")


def test_short_exact_integer_bitwise():
    B, D, T = 5, 211, 28
    rng = np.random.default_rng(4444)
    C = B * D
    x = {"a": rng.choice(np.array([-1.0, 0.0, 1.0, 1.0], dtype=np.float32), size=(C, T)),
         "b": rng.integers(-3, 4, size=(C, T)).astype(np.float32),
         "g": rng.integers(-3, 4, size=(C, T)).astype(np.float32),
         "h0": rng.integers(-3, 4, size=C).astype(np.float32)}
    got = run_scan(x, B, D, T, "bdt")
    ref = oracle_scan(x)
    log("short exact-integer")
    for k in ("h", "da", "db", "dh0"):
        assert np.array_equal(got[k], ref[k].astype(np.float32)), k
