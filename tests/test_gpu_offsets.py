"""Arrays that start one element past a 16-byte boundary.  The library takes
16-byte (and, for two channels per lane, 4- or 8-byte) vector accesses only
where every array it touches is aligned for them, and falls back to element
accesses otherwise; these tests hand every entry point views that begin one
element into a buffer (aligned to the element, not to the vector) and check
the results against the oracle at the usual bars, and against the same call
on aligned copies of the same values."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, bf16_dev, from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def shifted(t: torch.Tensor) -> torch.Tensor:
    """A copy of t that starts one element after a 256-byte aligned allocation."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def shifted_empty(t: torch.Tensor) -> torch.Tensor:
    return shifted(torch.zeros_like(t))


def close(x: torch.Tensor, y: torch.Tensor, tol: float) -> float:
    e = relerr(x.double().cpu().numpy(), y.double().cpu().numpy())
    assert e <= tol, e
    return e


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout,B,D,T", [("bdt", 2, 3, 4100), ("bdt", 1, 3, 20000),
                                          ("bdt", 3, 5, 40), ("tbd", 2, 70, 300)])
def test_scan_shifted(dtype, layout, B, D, T):
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd" if dtype == "f32" else "scan_fwd_bwd_bf16"], B=B, D=D,
                 T=T, seed=24000 + T + D)
    x = I.scan_inputs(w) if dtype == "f32" else I.scan_inputs_bf16(w)
    tol = 1e-5 if dtype == "f32" else 2e-2
    if dtype == "f32":
        vals = {k: x[k].astype(np.float32).astype(np.float64) for k in ("a", "b", "g")}
        dev = {k: to_dev(x[k].astype(np.float32), B, D, T, layout) for k in ("a", "b", "g")}
    else:
        bits = {k: x[k] for k in ("a", "b", "g")}
        vals = {k: I.bf16_bits_to_f64(v) for k, v in bits.items()}
        dev = {k: to_dev(np.ascontiguousarray(v).view(np.int16), B, D, T, layout).view(torch.bfloat16)
               for k, v in bits.items()}
    h0 = torch.from_numpy(x["h0"].astype(np.float32).reshape(B, D)).to(DEV)
    sa, sb, sg = (shifted(dev[k]) for k in ("a", "b", "g"))
    h = lrs.scan_fwd(sa, sb, h0, layout=layout, out=shifted_empty(dev["a"]))
    da, db, dh0 = lrs.scan_bwd(sa, h, sg, h0, layout=layout, grad_a=shifted_empty(dev["a"]),
                               grad_b=shifted_empty(dev["a"]))
    h_al = lrs.scan_fwd(dev["a"], dev["b"], h0, layout=layout)
    da_al, db_al, dh0_al = lrs.scan_bwd(dev["a"], h_al, dev["g"], h0, layout=layout)
    torch.cuda.synchronize()
    h64 = from_dev(h.float(), B, D, T, layout).astype(np.float64)
    h0_64 = x["h0"].astype(np.float32).astype(np.float64).reshape(-1)
    ref_h = oracle.scan_fwd(vals["a"], vals["b"], h0_64)
    ref_da, ref_db, ref_dh0 = oracle.scan_bwd(vals["a"], h64, h0_64, vals["g"])
    e = {"h": relerr(h64, ref_h),
         "da": relerr(from_dev(da.float(), B, D, T, layout).astype(np.float64), ref_da),
         "db": relerr(from_dev(db.float(), B, D, T, layout).astype(np.float64), ref_db),
         "dh0": relerr(dh0.cpu().numpy().reshape(-1).astype(np.float64), ref_dh0)}
    same = all(torch.equal(p, q) for p, q in ((h, h_al), (da, da_al), (db, db_al), (dh0, dh0_al)))
    log(f"shifted scan {dtype} {layout} {B}x{D}x{T}: " + ", ".join(f"{k}={v:.2e}" for k, v in e.items())
        + f"; bitwise equal to the aligned call: {same}")
    assert e["h"] <= tol and e["da"] <= tol and e["db"] <= tol and e["dh0"] <= 1e-5
    assert same


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_sru_shifted(io):
    B, D, T = 2, 96, 200
    w = I.scaled(I.WORKLOADS["sru_fwd_bwd"], B=B, D=D, T=T, seed=24100)
    s = I.sru_inputs(w)
    gh_bits = I.sru_grad_inputs(w)["gh"]
    z64 = {k: I.bf16_bits_to_f64(s[k]) for k in ("zf", "zr", "zx")}
    g64 = I.bf16_bits_to_f64(gh_bits)
    if io == "bf16":
        z = {k: bf16_dev(s[k]) for k in ("zf", "zr", "zx")}
        gh = bf16_dev(gh_bits)
    else:
        z = {k: torch.from_numpy(z64[k].astype(np.float32)).to(DEV) for k in z64}
        gh = torch.from_numpy(g64.astype(np.float32)).to(DEV)
    bf, br = (torch.from_numpy(s[k]).to(DEV) for k in ("bias_f", "bias_r"))
    zs = {k: shifted(v) for k, v in z.items()}
    cs = shifted(torch.zeros((T, B, D), device=DEV))
    h = lrs.sru_fwd(zs["zf"], zs["zr"], zs["zx"], bf, br, out=shifted_empty(z["zf"]), c_states=cs)
    outs = (shifted_empty(z["zf"]), shifted_empty(z["zf"]), shifted_empty(z["zf"]),
            torch.empty(D, device=DEV), torch.empty(D, device=DEV), torch.empty((B, D), device=DEV))
    g = lrs.sru_bwd(zs["zf"], zs["zr"], zs["zx"], bf, br, cs, shifted(gh), out=outs)
    cs_al = torch.empty((T, B, D), device=DEV)
    h_al = lrs.sru_fwd(z["zf"], z["zr"], z["zx"], bf, br, c_states=cs_al)
    g_al = lrs.sru_bwd(z["zf"], z["zr"], z["zx"], bf, br, cs_al, gh)
    torch.cuda.synchronize()
    ref_h, _ = oracle.sru_fwd(z64["zf"], z64["zr"], z64["zx"], s["bias_f"], s["bias_r"])
    tol = 2e-2 if io == "bf16" else 1e-5
    eh = relerr(h.double().cpu().numpy(), ref_h)
    assert eh <= tol
    # the backward against the aligned call (which the SRU backward tests pin to the oracle)
    for p, q, t in zip(g, g_al, (tol, tol, tol, 1e-5, 1e-5, 1e-5)):
        close(p, q, t)
    same = torch.equal(h, h_al) and torch.equal(cs, cs_al) and all(torch.equal(p, q) for p, q in zip(g, g_al))
    log(f"shifted sru {io}: h={eh:.2e}; bitwise equal to the aligned call: {same}")
    assert same


def test_lstm_shifted():
    B, D, T = 2, 96, 150
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=B, D=D, T=T, seed=24200)
    x = I.lstm_inputs(w)
    z = {k: bf16_dev(x[k]) for k in ("zf", "zi", "zc", "zo")}
    gh = bf16_dev(I.sru_grad_inputs(w)["gh"])
    zs = {k: shifted(v) for k, v in z.items()}
    cs = shifted(torch.zeros((T, B, D), device=DEV))
    h = lrs.lstm_fwd(zs["zf"], zs["zi"], zs["zc"], zs["zo"], out=shifted_empty(z["zf"]), c_states=cs)
    g = lrs.lstm_bwd(zs["zf"], zs["zi"], zs["zc"], zs["zo"], cs, shifted(gh))
    cs_al = torch.empty((T, B, D), device=DEV)
    h_al = lrs.lstm_fwd(z["zf"], z["zi"], z["zc"], z["zo"], c_states=cs_al)
    g_al = lrs.lstm_bwd(z["zf"], z["zi"], z["zc"], z["zo"], cs_al, gh)
    torch.cuda.synchronize()
    z64 = [I.bf16_bits_to_f64(x[k]) for k in ("zf", "zi", "zc", "zo")]
    ref_h, _ = oracle.lstm_fwd(*z64)
    eh = relerr(h.double().cpu().numpy(), ref_h)
    same = torch.equal(h, h_al) and torch.equal(cs, cs_al) and all(
        (p is None and q is None) or torch.equal(p, q) for p, q in zip(g, g_al))
    log(f"shifted lstm bf16: h={eh:.2e}; bitwise equal to the aligned call: {same}")
    assert eh <= 2e-2 and same


@pytest.mark.parametrize("T", [500, 8192, 20001])
def test_deer_shifted(T):
    B, D = 2, 3
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=24300 + T)
    x = I.deer_inputs(w)
    u = torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV)
    wd = torch.from_numpy(x["w"]).to(DEV)
    h, info = lrs.deer_solve(wd, shifted(u), out=shifted_empty(u))
    h_al, info_al = lrs.deer_solve(wd, u)
    torch.cuda.synchronize()
    ref_h, ref_it, _ = oracle.deer(x["w"], x["u"].reshape(B, D, T), x["h0"].reshape(B, D), None)
    e = relerr(h.double().cpu().numpy(), ref_h)
    log(f"shifted deer T={T}: h={e:.2e}, iterations {info['iters']} (oracle {ref_it}); "
        f"bitwise equal to the aligned call: {torch.equal(h, h_al)}")
    assert e <= 1e-5 and info["iters"] == ref_it == info_al["iters"]
    assert torch.equal(h, h_al)
