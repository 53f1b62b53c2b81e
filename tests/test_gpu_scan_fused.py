"""GPU parity of lrs_scan_fwd_bwd (forward and backward scan in one call)
against the fp64 oracle, to the fp32 bar 1e-5 on every output: ragged shapes
around every single-workgroup chunk size (one kernel) and beyond (the two
passes), without h (the backward with the forward recomputed), with grad_b
written over grad_h, the headline B=8 D=512 T=4096 shape, the streaming
variant, and exact integer inputs that must match bit for bit."""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from gpu_util import DEV, from_dev, log, to_dev
from test_gpu_scan import compare, oracle_scan

pytestmark = pytest.mark.gpu


def run_fused(x, B, D, T, layout="bdt", want_h=True, in_place=False):
    a = to_dev(x["a"], B, D, T, layout)
    b = to_dev(x["b"], B, D, T, layout)
    g = to_dev(x["g"], B, D, T, layout)
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    out = None
    if in_place:
        out = (torch.empty_like(a) if want_h else None, torch.empty_like(a), g,
               torch.empty((B, D), dtype=torch.float32, device=DEV))
    h, da, db, dh0 = lrs.scan_fwd_bwd(a, b, g, h0, layout=layout, want_h=want_h, out=out)
    torch.cuda.synchronize()
    if in_place:
        assert db.data_ptr() == g.data_ptr()
    got = {"da": from_dev(da, B, D, T, layout), "db": from_dev(db, B, D, T, layout),
           "dh0": dh0.cpu().numpy().reshape(-1)}
    if want_h:
        got["h"] = from_dev(h, B, D, T, layout)
    return got


SHAPES = [(1, 1, 1), (1, 3, 2), (2, 3, 5), (1, 7, 255), (1, 4, 256), (2, 5, 257), (3, 5, 1000),
          (1, 64, 1023), (1, 6, 1024), (1, 6, 2048), (2, 33, 4095), (1, 17, 4096),
          (1, 9, 4097), (2, 3, 8191), (2, 3, 8192), (1, 2, 8193), (1, 5, 12345), (3, 100, 129),
          (1, 257, 64)]


@pytest.mark.parametrize("B,D,T", SHAPES)
def test_fused_ragged(B, D, T):
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9000 + B * 131 + D * 7 + T)
    x = I.scan_inputs(w)
    compare(run_fused(x, B, D, T), oracle_scan(x), tag=f"fused/{B}x{D}x{T}")


@pytest.mark.parametrize("B,D,T", [(1, 3, 77), (2, 9, 4093), (1, 4, 8192)])
def test_fused_without_h_and_in_place(B, D, T):
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9100 + T)
    x = I.scan_inputs(w)
    ref = oracle_scan(x)
    del ref["h"]
    compare(run_fused(x, B, D, T, want_h=False, in_place=True), ref, tag=f"fused-noh/{B}x{D}x{T}")


@pytest.mark.parametrize("B,D,T", [(2, 5, 300), (1, 3, 20000)])
def test_two_pass_forms(B, D, T):
    """[T,B,D] layout and channels longer than 8192 steps run the two passes."""
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9200 + T)
    x = I.scan_inputs(w)
    for layout in ("bdt", "tbd"):
        compare(run_fused(x, B, D, T, layout=layout), oracle_scan(x),
                tag=f"fused-2pass/{layout}/{B}x{D}x{T}")


def test_fused_workload():
    w = I.WORKLOADS["scan_fwd_bwd"]
    log(f"fused scan_fwd_bwd B={w.B} D={w.D} T={w.T}")
    x = I.scan_inputs(w)
    compare(run_fused(x, w.B, w.D, w.T), oracle_scan(x), tag="fused/scan_fwd_bwd")


def test_fused_streamed():
    """16384 channels of 4096 steps (1.5 GiB in all): the nontemporal variant.
    Sampled channels against the oracle."""
    B, D, T = 16, 1024, 4096
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=9300)
    log(f"fused streamed B={B} D={D} T={T}")
    x = I.scan_inputs(w)
    a, b, g = (to_dev(x[k], B, D, T, "bdt") for k in ("a", "b", "g"))
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    h, da, db, dh0 = lrs.scan_fwd_bwd(a, b, g, h0)
    torch.cuda.synchronize()
    C = B * D
    sample = [0, 1, 77, 4095, 4096, 9000, C - 2, C - 1]
    ref = oracle_scan({k: x[k][sample] for k in ("a", "b", "g", "h0")})
    got = {"h": h.view(C, T)[sample].cpu().numpy(), "da": da.view(C, T)[sample].cpu().numpy(),
           "db": db.view(C, T)[sample].cpu().numpy(), "dh0": dh0.view(-1)[sample].cpu().numpy()}
    compare(got, ref, tag="fused/streamed")


def test_fused_exact_integer_bitwise():
    """a in {-1, 0, 1} and small integers elsewhere: every partial result is an
    exact fp32 integer, so the single kernel must match the oracle bit for bit."""
    B, D, T = 2, 7, 8192
    rng = np.random.default_rng(4343)
    x = {"a": rng.choice(np.array([-1.0, 0.0, 1.0, 1.0, 1.0], dtype=np.float32), size=(B * D, T)),
         "b": rng.integers(-2, 3, size=(B * D, T)).astype(np.float32),
         "g": rng.integers(-2, 3, size=(B * D, T)).astype(np.float32),
         "h0": rng.integers(-3, 4, size=B * D).astype(np.float32)}
    got = run_fused(x, B, D, T)
    ref = oracle_scan(x)
    assert np.max(np.abs(ref["h"])) < 2 ** 24 and np.max(np.abs(ref["db"])) < 2 ** 24
    for k in ("h", "da", "db", "dh0"):
        assert np.array_equal(got[k], ref[k].astype(np.float32)), k
