"""Million-step channels: the long forward + backward scan workload
(B=2, D=256, T=2^20, fp32, [B,D,T]) compared element by element with the fp64
oracle on every one of its 512 channels, and exact-integer inputs at the same
shape in both layouts that must match the oracle bit for bit.

Every channel crosses 128 forward and 64 backward look-back chunks ([B,D,T]),
or 8192 time blocks ([T,B,D]), so these tests cover the carry between
workgroups at full scale: tens of thousands of chunks in flight over all
eight XCDs.  The carry rule combines chunks in a fixed order, so repeated runs
must also agree bit for bit.

The oracle runs over 32-channel batches on the host (fp64), and the
comparison itself is done on the device against the uploaded fp64 reference,
so host memory stays bounded and the test takes seconds per batch."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu
TOL = 1e-5
BATCH = 32  # channels per oracle batch


def relerr_dev(got: torch.Tensor, ref: np.ndarray) -> float:
    """max |got - ref| / (1 + |ref|) with got on the device, ref fp64 on the host."""
    r = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64)).to(got.device)
    return ((got.double() - r).abs() / (1.0 + r.abs())).max().item()


def equal_dev(got: torch.Tensor, ref: np.ndarray) -> bool:
    """got (fp32, device) equals ref (fp64 holding exact fp32 values) bit for bit."""
    r = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float32)).to(got.device)
    return torch.equal(got.contiguous(), r)


def upload(x_ct: np.ndarray, B: int, D: int, T: int, layout: str) -> torch.Tensor:
    """[C, T] host array -> device [B,D,T] or [T,B,D]; the transpose is done on
    the device (data movement only)."""
    d = torch.from_numpy(np.ascontiguousarray(x_ct)).to(DEV)
    return d.view(B, D, T) if layout == "bdt" else d.t().contiguous().view(T, B, D)


def rows_of(t: torch.Tensor, C: int, T: int, layout: str) -> torch.Tensor:
    return t.view(C, T) if layout == "bdt" else t.view(T, C).t()


def run_fwd_bwd(a, b, g, layout):
    h = lrs.scan_fwd(a, b, None, layout=layout)
    da, db, dh0 = lrs.scan_bwd(a, h, g, None, layout=layout)
    torch.cuda.synchronize()
    return {"h": h, "da": da, "db": db, "dh0": dh0}


def check_all_channels(x, got, C, T, layout, exact=False, tag=""):
    """Oracle over every channel in batches; relative error bar or bitwise."""
    worst = {"h": 0.0, "da": 0.0, "db": 0.0, "dh0": 0.0}
    peak = 0.0
    for lo in range(0, C, BATCH):
        sl = slice(lo, min(C, lo + BATCH))
        ref_h = oracle.scan_fwd(x["a"][sl], x["b"][sl], None)
        ref_da, ref_db, ref_dh0 = oracle.scan_bwd(x["a"][sl], ref_h, None, x["g"][sl])
        ref = {"h": ref_h, "da": ref_da, "db": ref_db}
        for k, r in ref.items():
            dev = rows_of(got[k], C, T, layout)[sl]
            if exact:
                peak = max(peak, float(np.max(np.abs(r))))
                assert peak < 2 ** 24, f"{tag}: inputs not exact in fp32 ({k} reaches {peak})"
                assert equal_dev(dev, r), f"{tag}: {k} differs from the oracle, channels {sl}"
            else:
                worst[k] = max(worst[k], relerr_dev(dev, r))
        dh0 = got["dh0"].view(-1)[sl]
        if exact:
            assert equal_dev(dh0, ref_dh0), f"{tag}: dh0 differs, channels {sl}"
        else:
            worst["dh0"] = max(worst["dh0"], relerr_dev(dh0, ref_dh0))
    if exact:
        log(f"{tag}: all {C} channels bitwise equal to the oracle (largest |value| {peak:.0f})")
    else:
        log(f"{tag}: all {C} channels, errors " +
            ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
        for k, v in worst.items():
            assert v <= TOL, f"{tag}: {k} relerr {v:.3e} > {TOL}"


def test_scan_long_workload_every_channel():
    """The workload itself: h, dL/da, dL/db, dL/dh0 of all 512 channels within
    the 1e-5 bar; a second run gives the same bits; the adjoint identity
    <g, h> = <lam, b> (h0 = 0) holds per channel."""
    w = I.WORKLOADS["scan_long"]
    B, D, T = w.B, w.D, w.T
    C = B * D
    log(f"scan_long B={B} D={D} T={T}: generating inputs")
    x = I.scan_inputs(w)
    a, b, g = (upload(x[k], B, D, T, "bdt") for k in ("a", "b", "g"))
    log("scan_long: running on GPU (twice)")
    got = run_fwd_bwd(a, b, g, "bdt")
    again = run_fwd_bwd(a, b, g, "bdt")
    for k in got:
        assert torch.equal(got[k], again[k]), f"scan_long: {k} differs between two runs"
    del again
    log("scan_long: repeat run bitwise equal; comparing every channel with the oracle")
    check_all_channels(x, got, C, T, "bdt", tag="scan_long")
    lhs = (g.double() * got["h"].double()).sum(-1).view(-1)
    rhs = (got["db"].double() * b.double()).sum(-1).view(-1)
    rel = ((lhs - rhs).abs() / (1 + lhs.abs())).max().item()
    log(f"scan_long adjoint identity rel {rel:.2e}")
    assert rel < 1e-3


def exact_integer_inputs(C: int, T: int, seed: int) -> dict:
    """a in {-1, 0, 1} (zero with probability 2^-12, so a state runs on for
    thousands of steps across chunk boundaries; -1 with probability ~1/4),
    b and g in {-1, 0, 1}.  Every partial result is then a small integer,
    exact in fp32 whatever the association order."""
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 1 << 14, size=(C, T), dtype=np.int16)
    a = np.ones((C, T), dtype=np.float32)
    a[k < 4096] = -1.0
    a[k < 4] = 0.0
    del k
    b = rng.integers(-1, 2, size=(C, T), dtype=np.int8).astype(np.float32)
    g = rng.integers(-1, 2, size=(C, T), dtype=np.int8).astype(np.float32)
    return {"a": a, "b": b, "g": g}


@pytest.mark.parametrize("layout", ["bdt", "tbd"])
def test_scan_long_exact_integer_bitwise(layout):
    """Exact-integer inputs at the long workload's full shape: every output of
    every channel equals the oracle bit for bit, so no carry anywhere was
    dropped, duplicated, mis-ordered or read before it was published."""
    w = I.WORKLOADS["scan_long"]
    B, D, T = w.B, w.D, w.T
    C = B * D
    log(f"exact-integer long {layout} B={B} D={D} T={T}: generating inputs")
    x = exact_integer_inputs(C, T, 5151)
    a, b, g = (upload(x[k], B, D, T, layout) for k in ("a", "b", "g"))
    got = run_fwd_bwd(a, b, g, layout)
    del a, b, g
    log(f"exact-integer long {layout}: comparing every channel with the oracle")
    check_all_channels(x, got, C, T, layout, exact=True, tag=f"exact-integer long/{layout}")
