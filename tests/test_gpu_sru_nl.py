"""SRU with v_f * c_{t-1} in the forget gate, solved by DEER on the GPU
(lrs_sru_deer_fwd), against the fp64 oracle's DEER solve on identical
inputs: same iteration count, cell states to the fp32 bar 1e-5, h to the
I/O type's bar (1e-5 fp32, 2e-2 bf16); ragged shapes in both I/O types with
c0, v_f = 0 (one Newton step is the linear layer), the K_max cap, warm starts
(in place), the asynchronous form, and the full B=32 D=1024 T=2048 shape."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, bf16_dev, log

pytestmark = pytest.mark.gpu


def setup(w, io, vf=None):
    s = I.sru_inputs(w)
    z64 = {k: I.bf16_bits_to_f64(s[k]) for k in ("zf", "zr", "zx")}
    if io == "bf16":
        z = {k: bf16_dev(s[k]) for k in ("zf", "zr", "zx")}
    else:
        z = {k: torch.from_numpy(z64[k].astype(np.float32)).to(DEV) for k in z64}
    vf = I.sru_vf(w) if vf is None else vf
    p = {"bf": s["bias_f"], "br": s["bias_r"], "vf": vf}
    pd = {k: torch.from_numpy(v).to(DEV) for k, v in p.items()}
    return z, z64, p, pd


def run(w, io, c0=None, eps=1e-5, k_max=5, vf=None):
    z, z64, p, pd = setup(w, io, vf)
    c0d = None if c0 is None else torch.from_numpy(c0).to(DEV)
    h, cs, cl, info = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"], pd["vf"],
                                       c0d, eps=eps, k_max=k_max, want_c_last=True)
    torch.cuda.synchronize()
    hr, cr, it, dl = oracle.sru_deer(z64["zf"], z64["zr"], z64["zx"], p["bf"], p["br"], p["vf"],
                                     c0=c0, eps=eps, k_max=k_max)
    return (h.float().cpu().numpy(), cs.cpu().numpy(), cl.cpu().numpy(), info), (hr, cr, it, dl)


def check(got, ref, io, tag):
    (h, c, cl, info), (hr, cr, it, dl) = got, ref
    e = {"h": relerr(h, hr), "c": relerr(c, cr), "c_last": relerr(cl, cr[-1])}
    log(f"{tag}: iters {info['iters']} vs {it}, deltas {info['deltas']} vs {list(dl)}, "
        + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
    assert info["iters"] == it
    assert info["converged"] == (dl[-1] < 1e-5)
    assert e["c"] <= 1e-5 and e["c_last"] <= 1e-5
    assert e["h"] <= (2e-2 if io == "bf16" else 1e-5)


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (1, 3, 7), (2, 5, 64), (3, 50, 200),
                                   (1, 258, 513), (2, 128, 1000), (1, 64, 3000)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_sru_deer_ragged(B, D, T, io):
    w = I.scaled(I.WORKLOADS["sru_deer"], B=B, D=D, T=T, seed=10000 + B * 13 + D * 5 + T)
    c0 = np.random.default_rng(T + D).normal(size=(B, D)).astype(np.float32)
    check(*run(w, io, c0=c0, k_max=8), io, f"sru-deer {io} {B}x{D}x{T}")


def test_linear_case_matches_sru_layer():
    """v_f = 0: the first Newton step is the linear SRU cell state, the second
    changes nothing measurable, and h matches lrs_sru_fwd."""
    w = I.scaled(I.WORKLOADS["sru_deer"], B=2, D=96, T=700, seed=10100)
    z, _, p, pd = setup(w, "f32", vf=np.zeros(96, dtype=np.float32))
    h, cs, _, info = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"], pd["vf"])
    hl = lrs.sru_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"])
    torch.cuda.synchronize()
    log(f"linear case: {info}")
    assert info["iters"] == 2 and info["converged"]
    assert relerr(h.cpu().numpy(), hl.cpu().numpy()) < 1e-5


def test_kmax_cap_and_warm_start():
    """eps = 0 runs all K_max iterations (not converged), matching the oracle
    step for step; a start at the solution (in place) stops after one step."""
    w = I.scaled(I.WORKLOADS["sru_deer"], B=2, D=70, T=900, seed=10200)
    check(*run(w, "f32", eps=0.0, k_max=3), "f32", "sru-deer kmax")
    z, _, p, pd = setup(w, "f32")
    h, cs, _, info = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"], pd["vf"],
                                      k_max=10)
    first = cs.clone()
    h2, cs2, _, info2 = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"], pd["vf"],
                                         c_init=cs, c_states=cs, k_max=10)
    torch.cuda.synchronize()
    log(f"warm start: {info} then {info2}")
    assert cs2.data_ptr() == cs.data_ptr()
    assert info2["iters"] == 1 and info2["converged"]
    assert relerr(cs2.cpu().numpy(), first.cpu().numpy()) < 1e-5


def test_async_form_and_stats():
    w = I.scaled(I.WORKLOADS["sru_deer"], B=2, D=64, T=1500, seed=10300)
    z, _, p, pd = setup(w, "bf16")
    h1, c1, _, ref = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"], pd["vf"])
    h2, c2, _, ws = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"], pd["vf"],
                                     sync=False)
    st = lrs.deer_stats(ws, 5)
    torch.cuda.synchronize()
    assert st["iters"] == ref["iters"] and st["converged"] == ref["converged"]
    assert torch.equal(h1, h2) and torch.equal(c1, c2)


def test_sru_deer_workload():
    w = I.WORKLOADS["sru_deer"]
    log(f"sru_deer B={w.B} D={w.D} T={w.T}")
    got, ref = run(w, "bf16")
    check(got, ref, "bf16", "sru_deer workload")
    assert got[3]["iters"] == 5 and got[3]["converged"]
