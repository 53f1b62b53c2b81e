"""SRU backward on the GPU (lrs_sru_fwd saving the cell states, then
lrs_sru_bwd) against the fp64 oracle, on identical inputs: ragged shapes in
both I/O types with c0 and dL/dc_T, and the full B=32 D=1024 T=2048 shape.
Gradients written in the I/O type meet that type's bar (1e-5 fp32, 2e-2
bf16); the fp32 outputs (bias gradients, dL/dc0) meet 1e-5."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, bf16_dev, log

pytestmark = pytest.mark.gpu


def sru_bwd_case(w, io, c0=None, gcl=None):
    s = I.sru_inputs(w)
    g = I.sru_grad_inputs(w)
    B, D, T = w.B, w.D, w.T
    names = ("zf", "zr", "zx", "gh")
    src = dict(s, gh=g["gh"])
    z64 = {k: I.bf16_bits_to_f64(src[k]) for k in names}
    if io == "bf16":
        z = {k: bf16_dev(src[k]) for k in names}
    else:
        z = {k: torch.from_numpy(z64[k].astype(np.float32)).to(DEV) for k in names}
    bf = torch.from_numpy(s["bias_f"]).to(DEV)
    br = torch.from_numpy(s["bias_r"]).to(DEV)
    c0d = None if c0 is None else torch.from_numpy(c0).to(DEV)
    gcld = None if gcl is None else torch.from_numpy(gcl).to(DEV)
    cs = torch.empty((T, B, D), dtype=torch.float32, device=DEV)
    lrs.sru_fwd(z["zf"], z["zr"], z["zx"], bf, br, c0d, c_states=cs)
    got = lrs.sru_bwd(z["zf"], z["zr"], z["zx"], bf, br, cs, z["gh"], c0=c0d, grad_c_last=gcld)
    torch.cuda.synchronize()
    got = dict(zip(("dzf", "dzr", "dzx", "dbf", "dbr", "dc0"),
                   (t.float().cpu().numpy() for t in got)))
    ref = oracle.sru_bwd(z64["zf"], z64["zr"], z64["zx"], s["bias_f"], s["bias_r"], z64["gh"],
                         c0=c0, gcl=gcl)
    return got, ref


def check(got, ref, io, tag):
    errs = {k: relerr(got[k], ref[k]) for k in got}
    log(f"{tag}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        bar = 2e-2 if (io == "bf16" and k in ("dzf", "dzr", "dzx")) else 1e-5
        assert e <= bar, (k, e)


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (1, 2, 3), (2, 3, 65), (1, 6, 64), (3, 50, 200),
                                   (1, 258, 513), (2, 128, 1000), (1, 64, 4097)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_sru_bwd_ragged(B, D, T, io):
    w = I.scaled(I.WORKLOADS["sru_fwd_bwd"], B=B, D=D, T=T, seed=7000 + B * 13 + D * 5 + T)
    rng = np.random.default_rng(T + D)
    c0 = rng.normal(size=(B, D)).astype(np.float32)
    gcl = rng.normal(size=(B, D)).astype(np.float32)
    got, ref = sru_bwd_case(w, io, c0=c0, gcl=gcl)
    check(got, ref, io, f"sru bwd {io} B={B} D={D} T={T}")


def test_sru_bwd_workload():
    """B=32 D=1024 T=2048 bf16 (the streaming variants), c0 = 0, no dL/dc_T."""
    w = I.WORKLOADS["sru_fwd_bwd"]
    log(f"sru_fwd_bwd B={w.B} D={w.D} T={w.T}")
    got, ref = sru_bwd_case(w, "bf16")
    check(got, ref, "bf16", "sru_fwd_bwd")


def test_sru_bwd_deterministic_bias_sums():
    """The bias gradients are summed in a fixed order: two runs agree bit for bit."""
    w = I.scaled(I.WORKLOADS["sru_fwd_bwd"], B=4, D=96, T=700, seed=7100)
    a, _ = sru_bwd_case(w, "f32")
    b, _ = sru_bwd_case(w, "f32")
    assert np.array_equal(a["dbf"], b["dbf"]) and np.array_equal(a["dbr"], b["dbr"])


def test_sru_bwd_empty_time():
    """T = 0: the bias gradients are empty sums and dL/dc0 = dL/dc_T."""
    B, D = 2, 5
    e = torch.empty((0, B, D), dtype=torch.bfloat16, device=DEV)
    cs = torch.empty((0, B, D), dtype=torch.float32, device=DEV)
    bias = torch.zeros(D, device=DEV)
    gcl = torch.arange(B * D, dtype=torch.float32, device=DEV).reshape(B, D)
    out = (torch.empty_like(e), torch.empty_like(e), torch.empty_like(e),
           torch.full((D,), 7.0, device=DEV), torch.full((D,), 7.0, device=DEV),
           torch.full((B, D), 7.0, device=DEV))
    _, _, _, dbf, dbr, dc0 = lrs.sru_bwd(e, e, e, bias, bias, cs, e, grad_c_last=gcl, out=out)
    torch.cuda.synchronize()
    assert torch.equal(dbf, torch.zeros_like(dbf)) and torch.equal(dbr, torch.zeros_like(dbr))
    assert torch.equal(dc0, gcl)
