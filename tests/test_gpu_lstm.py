"""LSTM cell-state layer with input-only gates on the GPU (lrs_lstm_fwd, which
can save the cell states, then lrs_lstm_bwd) against the fp64 oracle on
identical inputs: ragged shapes in both I/O types with c0 and dL/dc_T, tiles
spanning several time blocks, and the full B=32 D=1024 T=2048 bf16 shape.
Values written in the I/O type meet that type's bar (1e-5 fp32, 2e-2 bf16);
the fp32 outputs (c_T, the saved cell states, dL/dc0) meet 1e-5."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, bf16_dev, log

pytestmark = pytest.mark.gpu

GATES = ("zf", "zi", "zc", "zo")


def dev_inputs(w, io):
    s = I.lstm_inputs(w)
    s["gh"] = I.sru_grad_inputs(w)["gh"]
    z64 = {k: I.bf16_bits_to_f64(v) for k, v in s.items()}
    if io == "bf16":
        z = {k: bf16_dev(v) for k, v in s.items()}
    else:
        z = {k: torch.from_numpy(v.astype(np.float32)).to(DEV) for k, v in z64.items()}
    return z, z64


def bar(io, k):
    return 2e-2 if io == "bf16" and k in ("h", "dzf", "dzi", "dzc", "dzo") else 1e-5


def check(errs, io, tag):
    log(f"{tag}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= bar(io, k), (k, e)


def run_case(w, io, c0=None, gcl=None, backward=True):
    z, z64 = dev_inputs(w, io)
    T, B, D = w.T, w.B, w.D
    c0d = None if c0 is None else torch.from_numpy(c0).to(DEV)
    gcld = None if gcl is None else torch.from_numpy(gcl).to(DEV)
    cs = torch.empty((T, B, D), dtype=torch.float32, device=DEV)
    h, c_last = lrs.lstm_fwd(z["zf"], z["zi"], z["zc"], z["zo"], c0d, want_c_last=True,
                             c_states=cs)
    got = {"h": h, "c_last": c_last, "cs": cs}
    if backward:
        g = lrs.lstm_bwd(z["zf"], z["zi"], z["zc"], z["zo"], cs, z["gh"], c0=c0d,
                         grad_c_last=gcld)
        got.update(zip(("dzf", "dzi", "dzc", "dzo", "dc0"), g))
    torch.cuda.synchronize()
    got = {k: v.float().cpu().numpy() for k, v in got.items()}
    h_ref, c_ref = oracle.lstm_fwd(*(z64[k] for k in GATES), c0=c0)
    # the oracle's cell states: c_T of every prefix is c_last of the prefix run
    errs = {"h": relerr(got["h"], h_ref), "c_last": relerr(got["c_last"], c_ref)}
    if T <= 64:
        cs_ref = np.stack([oracle.lstm_fwd(*(z64[k][: t + 1] for k in GATES), c0=c0)[1]
                           for t in range(T)])
        errs["cs"] = relerr(got["cs"], cs_ref)
    if backward:
        ref = oracle.lstm_bwd(*(z64[k] for k in GATES), z64["gh"], c0=c0, gcl=gcl)
        errs.update({k: relerr(got[k], ref[k]) for k in ("dzf", "dzi", "dzc", "dzo", "dc0")})
    return errs


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (1, 2, 3), (2, 3, 65), (1, 6, 64), (3, 50, 200),
                                   (1, 258, 513), (2, 128, 1000), (1, 64, 4097)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_lstm_ragged(B, D, T, io):
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=B, D=D, T=T, seed=8000 + B * 13 + D * 5 + T)
    rng = np.random.default_rng(T + 3 * D)
    c0 = rng.normal(size=(B, D)).astype(np.float32)
    gcl = rng.normal(size=(B, D)).astype(np.float32)
    check(run_case(w, io, c0=c0, gcl=gcl), io, f"lstm {io} B={B} D={D} T={T}")


def test_lstm_saved_states_exact_prefix():
    """The saved cell states at T=40 match the oracle's c_T of every prefix."""
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=2, D=70, T=40, seed=8100)
    check(run_case(w, "f32", backward=False), "f32", "lstm saved states")


def test_lstm_workload():
    """B=32 D=1024 T=2048 bf16 (streaming variants), c0 = 0, no dL/dc_T."""
    w = I.WORKLOADS["lstm_fwd_bwd"]
    log(f"lstm_fwd_bwd B={w.B} D={w.D} T={w.T}")
    check(run_case(w, "bf16"), "bf16", "lstm_fwd_bwd")


def test_lstm_forward_without_saving_matches():
    """Leaving out c_states (another launch plan) does not change h or c_T."""
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=4, D=96, T=700, seed=8200)
    z, _ = dev_inputs(w, "bf16")
    cs = torch.empty((w.T, w.B, w.D), dtype=torch.float32, device=DEV)
    h1, c1 = lrs.lstm_fwd(z["zf"], z["zi"], z["zc"], z["zo"], want_c_last=True, c_states=cs)
    h2, c2 = lrs.lstm_fwd(z["zf"], z["zi"], z["zc"], z["zo"], want_c_last=True)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(c1, c2)


def test_lstm_empty_time():
    """T = 0: c_T = c0 and dL/dc0 = dL/dc_T."""
    B, D = 2, 5
    e = torch.empty((0, B, D), dtype=torch.bfloat16, device=DEV)
    cs = torch.empty((0, B, D), dtype=torch.float32, device=DEV)
    c0 = torch.arange(B * D, dtype=torch.float32, device=DEV).reshape(B, D)
    _, c_last = lrs.lstm_fwd(e, e, e, e, c0, want_c_last=True)
    *_, dc0 = lrs.lstm_bwd(e, e, e, e, cs, e, grad_c_last=c0 + 1)
    torch.cuda.synchronize()
    assert torch.equal(c_last, c0) and torch.equal(dc0, c0 + 1)
