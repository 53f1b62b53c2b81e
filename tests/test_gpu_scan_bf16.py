"""Linear scan with bf16 arrays (a, b, h, dL/dh, dL/da, dL/db in bf16; h0 and
dL/dh0 fp32; state and arithmetic fp32) against the fp64 oracle run on the
exact bf16 values the GPU receives.

Every kernel family is reached: sequential (T <= 4) and packed (T <= 64)
short channels, single-chunk channels, multi-chunk channels with the
look-back (forward chunks of 8192 steps, backward chunks of 16384), the
one-kernel forward+backward, and the [T,B,D] tiles, with ragged T and ragged
channel counts.  The bar is max|gpu-oracle|/(1+|oracle|) <= 2e-2 for bf16
outputs and 1e-5 for the fp32 dL/dh0.  The backward is checked against the
oracle fed the GPU's own bf16 h, the input it actually consumed.

Exact-integer inputs (a in {-1,0,1}, b and dL/dh in {-1,0,1}) keep every fp32
intermediate an exact integer, so the rounded bf16 outputs must equal the
oracle's exact results rounded to bf16 (nearest-even) bit for bit, across
chunk and time-block boundaries in both layouts."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, from_dev, log, to_dev

pytestmark = pytest.mark.gpu
TOL16, TOL32 = 2e-2, 1e-5


def up16(bits_ct, B, D, T, layout):
    """bf16 bit patterns [C, T] -> device bf16 tensor in the layout."""
    return to_dev(np.ascontiguousarray(bits_ct).view(np.int16), B, D, T, layout).view(torch.bfloat16)


def down16(t, B, D, T, layout):
    """device bf16 tensor -> ([C, T] bit patterns, the same values in fp64)."""
    bits = from_dev(t.view(torch.int16), B, D, T, layout).view(np.uint16)
    return bits, I.bf16_bits_to_f64(bits)


def bf16_case(B, D, T, seed):
    """The bf16 scan recipe (each value rounded once from its fp64 draw)."""
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd_bf16"], B=B, D=D, T=T, seed=seed)
    x = I.scan_inputs_bf16(w)
    bits = {k: x[k] for k in ("a", "b", "g")}
    vals = {k: I.bf16_bits_to_f64(v) for k, v in bits.items()}
    h0 = x["h0"].astype(np.float32)
    return bits, vals, h0


SHAPES = [(1, 1, 1), (2, 3, 4), (3, 5, 33), (4, 7, 64), (2, 37, 200), (1, 130, 1001),
          (2, 64, 4096), (1, 3, 8193), (2, 5, 20001), (1, 2, 50000)]


@pytest.mark.parametrize("B,D,T", SHAPES)
@pytest.mark.parametrize("layout", ["bdt", "tbd"])
def test_scan_bf16_fwd_bwd(B, D, T, layout):
    bits, vals, h0 = bf16_case(B, D, T, 20000 + 7 * B + 3 * D + T)
    a, b, g = (up16(bits[k], B, D, T, layout) for k in ("a", "b", "g"))
    h0d = torch.from_numpy(h0.reshape(B, D)).to(DEV)
    h = lrs.scan_fwd(a, b, h0d, layout=layout)
    da, db, dh0 = lrs.scan_bwd(a, h, g, h0d, layout=layout)
    torch.cuda.synchronize()
    assert h.dtype == da.dtype == db.dtype == torch.bfloat16 and dh0.dtype == torch.float32
    _, h64 = down16(h, B, D, T, layout)
    ref_h = oracle.scan_fwd(vals["a"], vals["b"], h0.astype(np.float64).reshape(-1))
    ref_da, ref_db, ref_dh0 = oracle.scan_bwd(vals["a"], h64, h0.astype(np.float64).reshape(-1),
                                              vals["g"])
    e = {"h": relerr(h64, ref_h),
         "da": relerr(down16(da, B, D, T, layout)[1], ref_da),
         "db": relerr(down16(db, B, D, T, layout)[1], ref_db),
         "dh0": relerr(dh0.cpu().numpy().reshape(-1), ref_dh0)}
    log(f"bf16 scan {layout} {B}x{D}x{T}: " + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
    assert e["h"] <= TOL16 and e["da"] <= TOL16 and e["db"] <= TOL16
    assert e["dh0"] <= TOL32


@pytest.mark.parametrize("B,D,T", [(2, 3, 4), (3, 5, 33), (2, 37, 200), (1, 130, 1001),
                                   (2, 64, 4096), (1, 3, 8192), (1, 3, 8193)])
def test_scan_bf16_fwd_bwd_one_call(B, D, T):
    """lrs_scan_fwd_bwd with bf16 arrays ([B,D,T]): one kernel for single-chunk
    channels (h stays fp32 between the passes), the two passes otherwise;
    also with grad_b written over grad_h."""
    bits, vals, h0 = bf16_case(B, D, T, 21000 + 5 * B + D + T)
    a, b, g = (up16(bits[k], B, D, T, "bdt") for k in ("a", "b", "g"))
    h0d = torch.from_numpy(h0.reshape(B, D)).to(DEV)
    h64ref = oracle.scan_fwd(vals["a"], vals["b"], h0.astype(np.float64).reshape(-1))
    ref_da, ref_db, ref_dh0 = oracle.scan_bwd(vals["a"], h64ref, h0.astype(np.float64).reshape(-1),
                                              vals["g"])
    for in_place in (False, True):
        gg = g.clone()
        out = (torch.empty_like(a), torch.empty_like(a), gg if in_place else torch.empty_like(a),
               torch.empty((B, D), device=DEV))
        h, da, db, dh0 = lrs.scan_fwd_bwd(a, b, gg, h0d, out=out)
        torch.cuda.synchronize()
        # the two-pass form consumes the rounded h: give the oracle the same
        _, h64 = down16(h, B, D, T, "bdt")
        r_da, r_db, r_dh0 = (ref_da, ref_db, ref_dh0) if T <= 8192 else \
            oracle.scan_bwd(vals["a"], h64, h0.astype(np.float64).reshape(-1), vals["g"])
        e = {"h": relerr(h64, h64ref),
             "da": relerr(down16(da, B, D, T, "bdt")[1], r_da),
             "db": relerr(down16(db, B, D, T, "bdt")[1], r_db),
             "dh0": relerr(dh0.cpu().numpy().reshape(-1), r_dh0)}
        log(f"bf16 fwd+bwd {B}x{D}x{T} in_place={in_place}: "
            + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
        assert e["h"] <= TOL16 and e["da"] <= TOL16 and e["db"] <= TOL16
        assert e["dh0"] <= TOL32


def integer_case(C, T, seed):
    """a in {-1, 0, 1} with a zero every 8 steps on average (states stay small
    integers), b and dL/dh in {-1, 0, 1}: every value exact in bf16 and fp32."""
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 8, size=(C, T))
    a = np.where(k == 0, 0.0, np.where(k < 3, -1.0, 1.0))
    b = rng.integers(-1, 2, size=(C, T)).astype(np.float64)
    g = rng.integers(-1, 2, size=(C, T)).astype(np.float64)
    return a, b, g


@pytest.mark.parametrize("B,D,T,layout", [(1, 3, 40000, "bdt"), (2, 5, 9000, "bdt"),
                                          (1, 130, 3000, "tbd"), (2, 70, 20001, "tbd")])
def test_scan_bf16_exact_integer_bitwise(B, D, T, layout):
    C = B * D
    a, b, g = integer_case(C, T, 22000 + T)
    ad, bd, gd = (up16(I.to_bf16_bits(x), B, D, T, layout) for x in (a, b, g))
    h = lrs.scan_fwd(ad, bd, None, layout=layout)
    da, db, dh0 = lrs.scan_bwd(ad, h, gd, None, layout=layout)
    torch.cuda.synchronize()
    hb, h64 = down16(h, B, D, T, layout)
    ref_h = oracle.scan_fwd(a, b, None)
    assert np.array_equal(hb, I.to_bf16_bits(ref_h)), "h differs from the oracle"
    ref_da, ref_db, ref_dh0 = oracle.scan_bwd(a, h64, None, g)
    assert np.max(np.abs(ref_da)) < 2 ** 24 and np.max(np.abs(ref_db)) < 2 ** 24
    assert np.array_equal(down16(da, B, D, T, layout)[0], I.to_bf16_bits(ref_da)), "dL/da differs"
    assert np.array_equal(down16(db, B, D, T, layout)[0], I.to_bf16_bits(ref_db)), "dL/db differs"
    assert np.array_equal(dh0.cpu().numpy().reshape(-1).astype(np.float64), ref_dh0), "dL/dh0 differs"
    log(f"bf16 exact-integer {layout} {B}x{D}x{T}: bitwise equal (largest |h| "
        f"{np.max(np.abs(ref_h)):.0f}, |dL/da| {np.max(np.abs(ref_da)):.0f})")


def test_scan_bf16_workload_shape_sampled():
    """B=8 D=512 T=4096 with bf16 arrays in both layouts: 16 sampled channels
    against the oracle, every element of h and dL/db finite."""
    B, D, T = 8, 512, 4096
    bits, vals, h0 = bf16_case(B, D, T, 23000)
    rows = np.arange(0, B * D, B * D // 16)
    for layout in ("bdt", "tbd"):
        a, b, g = (up16(bits[k], B, D, T, layout) for k in ("a", "b", "g"))
        h0d = torch.from_numpy(h0.reshape(B, D)).to(DEV)
        h = lrs.scan_fwd(a, b, h0d, layout=layout)
        da, db, dh0 = lrs.scan_bwd(a, h, g, h0d, layout=layout)
        torch.cuda.synchronize()
        _, h64 = down16(h, B, D, T, layout)
        _, db64 = down16(db, B, D, T, layout)
        assert np.isfinite(h64).all() and np.isfinite(db64).all()
        ref_h = oracle.scan_fwd(vals["a"][rows], vals["b"][rows], h0.reshape(-1)[rows].astype(np.float64))
        ref_da, ref_db, _ = oracle.scan_bwd(vals["a"][rows], h64[rows],
                                            h0.reshape(-1)[rows].astype(np.float64), vals["g"][rows])
        eh = relerr(h64[rows], ref_h)
        edb = relerr(db64[rows], ref_db)
        eda = relerr(down16(da, B, D, T, layout)[1][rows], ref_da)
        log(f"bf16 scan workload shape {layout}: sampled h={eh:.2e} da={eda:.2e} db={edb:.2e}")
        assert eh <= TOL16 and eda <= TOL16 and edb <= TOL16


def test_scan_long_bf16_every_channel():
    """The bf16 long workload (B=2, D=256, T=2^20, [B,D,T], 128 forward and 64
    backward look-back chunks per channel): every one of its 512 channels
    against the oracle run on the bf16 values, in 32-channel batches compared
    on the device; a second run gives the same bits."""
    from test_gpu_scan_long import relerr_dev, rows_of, upload
    w = I.WORKLOADS["scan_long_bf16"]
    B, D, T = w.B, w.D, w.T
    C = B * D
    log(f"scan_long_bf16 B={B} D={D} T={T}: generating inputs")
    x = I.scan_inputs_bf16(w)
    a, b, g = (upload(x[k].view(np.int16), B, D, T, "bdt").view(torch.bfloat16)
               for k in ("a", "b", "g"))
    runs = []
    for _ in range(2):
        h = lrs.scan_fwd(a, b, None)
        da, db, dh0 = lrs.scan_bwd(a, h, g, None)
        torch.cuda.synchronize()
        runs.append({"h": h, "da": da, "db": db, "dh0": dh0})
    got, again = runs
    for k in got:
        assert torch.equal(got[k], again[k]), f"scan_long_bf16: {k} differs between two runs"
    del again, runs
    worst = {"h": 0.0, "da": 0.0, "db": 0.0, "dh0": 0.0}
    for lo in range(0, C, 32):
        sl = slice(lo, lo + 32)
        av, bv, gv = (I.bf16_bits_to_f64(x[k][sl]) for k in ("a", "b", "g"))
        h_dev = rows_of(got["h"], C, T, "bdt")[sl]
        worst["h"] = max(worst["h"], relerr_dev(h_dev, oracle.scan_fwd(av, bv, None)))
        h64 = h_dev.double().cpu().numpy()  # the bf16 h the backward consumed
        ref_da, ref_db, ref_dh0 = oracle.scan_bwd(av, h64, None, gv)
        worst["da"] = max(worst["da"], relerr_dev(rows_of(got["da"], C, T, "bdt")[sl], ref_da))
        worst["db"] = max(worst["db"], relerr_dev(rows_of(got["db"], C, T, "bdt")[sl], ref_db))
        worst["dh0"] = max(worst["dh0"], relerr_dev(got["dh0"].view(-1)[sl], ref_dh0))
    log("scan_long_bf16: all 512 channels, errors " + ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    assert worst["h"] <= TOL16 and worst["da"] <= TOL16 and worst["db"] <= TOL16
    assert worst["dh0"] <= TOL32
