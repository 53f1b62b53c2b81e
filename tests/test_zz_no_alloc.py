"""Allocation-free fused scan, lrs_scan_fwd_bwd_noalloc, called through the C
ABI: its look-back state lives in the library's fixed per-GPU array instead of
a workspace.  Its outputs must equal those of lrs_scan_fwd_bwd with a
workspace bit for bit (the same kernels, plan and fixed combine order), on two
calls in a row where the second is smaller (the array still holds the first
call's state), in both layouts and for fp32 and bf16 arrays, and match the fp64
oracle to the 1e-5 bar (fp32); a
single-workgroup shape needs no array; a shape beyond the array is rejected
before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import binding
from linear_recurrence_scan_diagonal_amd import inputs as I
from gpu_util import DEV, from_dev, log, to_dev
from test_gpu_scan import compare, oracle_scan

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(a, b, h0, g, layout):
    """lrs_scan_fwd_bwd_noalloc into fresh NaN-filled outputs."""
    lib = lrs.load()
    B, D, T = binding._dims(a, layout)
    h, ga, gb = (torch.full_like(a, float("nan")) for _ in range(3))
    gh0 = torch.full((B, D), float("nan"), device=a.device)
    rc = lib.lrs_scan_fwd_bwd_noalloc(_p(a), _p(b), _p(h0), _p(g), _p(h), _p(ga), _p(gb), _p(gh0),
                                      B, D, T, binding.LAYOUTS[layout], binding.DTYPES[a.dtype],
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == binding.LRS_OK, lib.lrs_status_string(rc)
    return h, ga, gb, gh0


def one_call(layout, B, D, T, seed):
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=seed)
    x = I.scan_inputs(w)
    a, b, g = (to_dev(x[k], B, D, T, layout) for k in ("a", "b", "g"))
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    need = lrs.scan_workspace_bytes(B, D, T, layout)
    log(f"noalloc {layout} B={B} D={D} T={T}: workspace form needs {need} bytes")
    assert need <= 8 << 20
    got = noalloc(a, b, h0, g, layout)
    ref = lrs.scan_fwd_bwd(a, b, g, h0, layout=layout)
    torch.cuda.synchronize()
    for name, u, v in zip(("h", "grad_a", "grad_b", "grad_h0"), got, ref):
        assert torch.equal(u, v), f"noalloc {layout} {B}x{D}x{T}: {name} differs"
    res = {"h": from_dev(got[0], B, D, T, layout), "da": from_dev(got[1], B, D, T, layout),
           "db": from_dev(got[2], B, D, T, layout), "dh0": got[3].cpu().numpy().reshape(-1)}
    compare(res, oracle_scan(x), tag=f"noalloc {layout} {B}x{D}x{T}")
    return need


@pytest.mark.parametrize("layout,big,small", [
    ("bdt", (2, 64, 300_000), (1, 5, 20_000)),   # 37 / 19 chunks, then 3 / 2
    ("tbd", (2, 128, 50_000), (1, 40, 3_000)),   # 391 time blocks, then 24
])
def test_noalloc_matches_workspace_form(layout, big, small):
    n1 = one_call(layout, *big, seed=18000 + big[2])
    n2 = one_call(layout, *small, seed=18000 + small[2])
    assert n1 > n2 > 0


@pytest.mark.parametrize("layout,big,small", [
    ("bdt", (2, 64, 300_000), (1, 5, 20_000)),
    ("tbd", (2, 128, 50_000), (1, 40, 3_000)),
])
def test_noalloc_bf16_matches_workspace_form(layout, big, small):
    """bf16 arrays (fp32 h0 and dL/dh0): the same two calls in a row, bit for
    bit the workspace form (whose bf16 parity with the oracle is tested with
    the other bf16 scans)."""
    for (B, D, T) in (big, small):
        w = I.scaled(I.WORKLOADS["scan_fwd_bwd_bf16"], B=B, D=D, T=T, seed=18200 + T)
        x = I.scan_inputs_bf16(w)
        a, b, g = (to_dev(x[k].view(np.int16), B, D, T, layout).view(torch.bfloat16)
                   for k in ("a", "b", "g"))
        h0 = torch.from_numpy(x["h0"].reshape(B, D).astype(np.float32)).to(DEV)
        got = noalloc(a, b, h0, g, layout)
        ref = lrs.scan_fwd_bwd(a, b, g, h0, layout=layout)
        torch.cuda.synchronize()
        log(f"noalloc bf16 {layout} B={B} D={D} T={T}")
        for name, u, v in zip(("h", "grad_a", "grad_b", "grad_h0"), got, ref):
            assert torch.equal(u, v), f"noalloc bf16 {layout} {B}x{D}x{T}: {name} differs"
        assert torch.isfinite(got[0].float()).all() and torch.isfinite(got[3]).all()


def test_noalloc_single_workgroup_shape():
    """Channels that fit one workgroup run the one-kernel form (no look-back
    state, no array needed)."""
    assert one_call("bdt", 2, 8, 1000, seed=18100) == 0


def test_noalloc_rejects_shape_beyond_the_array():
    """[T,B,D] with 2^28 elements needs 16 MiB of look-back state: rejected
    before any launch (the pointers are never touched)."""
    lib = lrs.load()
    B, D, T = 4, 1024, 1 << 16
    assert lrs.scan_workspace_bytes(B, D, T, "tbd") > 8 << 20
    p = ctypes.c_void_p(1 << 20)
    rc = lib.lrs_scan_fwd_bwd_noalloc(p, p, None, p, p, p, p, None, B, D, T,
                                      binding.LAYOUTS["tbd"], 0, None)
    assert rc == binding.LRS_ERR_WORKSPACE
