"""The fused DEER solve (all Newton iterations in one walk over each channel,
used for channels one workgroup walks and K_max <= 8) against the fp64 oracle
and against the one-launch-per-iteration path (plan option deer_fuse = 0) on the same
inputs: the full B=16 D=512 T=8192 shape, ragged and unaligned lengths,
h0 given, K_max = 1 and 8, and early stops (a large eps, a warm start near the
solution, the warm start held in h itself), where the pass's K_max iterations
are replaced by a recompute with exactly the iterations the stop rule allows."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def solve(x, B, D, T, eps, k_max, h_init=None, in_place=False):
    w = torch.from_numpy(x["w"]).to(DEV)
    u = torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV)
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    hi = None if h_init is None else torch.from_numpy(h_init.astype(np.float32)).to(DEV)
    h, info = lrs.deer_solve(w, u, h0, hi, eps=eps, k_max=k_max, out=hi if in_place else None)
    torch.cuda.synchronize()
    return h.cpu().numpy(), info


def both_paths(plan, x, B, D, T, eps, k_max, h_init=None, in_place=False):
    out = {}
    for mode, flag in (("fused", "1"), ("per-iteration", "0")):
        plan(deer_fuse=int(flag))
        out[mode] = solve(x, B, D, T, eps, k_max, h_init, in_place)
    return out


@pytest.mark.parametrize("B,D,T,eps,k_max,h0,warm,in_place", [
    (16, 512, 8192, 1e-5, 5, False, False, False),   # the DEER workload
    (2, 5, 8192, 1e-5, 5, True, False, False),       # two sub-chunks, h0
    (2, 3, 8190, 1e-5, 5, True, False, False),       # partial sub-chunk, T % 4 != 0
    (1, 7, 6001, 1e-5, 8, True, False, False),       # K_max = 8, odd length
    (3, 4, 4096, 1e-5, 1, True, False, False),       # K_max = 1 (one sub-chunk)
    (3, 4, 5000, 1e-5, 1, False, False, False),      # K_max = 1, two sub-chunks
    (2, 6, 8192, 1e-2, 6, True, False, False),       # early stop: recomputed
    (2, 6, 7777, 1e-5, 6, True, True, False),        # warm start, early stop
    (2, 6, 8192, 1e-5, 6, True, True, True),         # warm start held in h, early stop
    (2, 6, 3000, 1e-5, 3, True, True, True),         # warm start in h, stops at K_max
    (1, 1, 1, 1e-5, 5, True, False, False),          # one step
    (2, 3, 512, 1e-5, 5, True, False, False),        # longest channel of 4 steps per lane
    (2, 3, 513, 1e-5, 5, True, True, False),         # one wave of 8 steps per lane, partial
    (1, 4, 1024, 1e-5, 5, True, False, False),       # one wave of 2 rows of 8 steps, full
    (2, 3, 1500, 1e-2, 6, True, False, False),       # two waves, partial, early stop
    (2, 3, 2048, 1e-5, 5, True, False, False),       # two waves of 2 rows of 8 steps, full
    (2, 3, 2049, 1e-5, 5, True, True, False),        # four waves, partial
    (2, 3, 4097, 1e-5, 5, True, False, False),       # second sub-chunk of one step
    (2, 3, 16384, 1e-5, 5, True, False, False),      # four sub-chunks (forced: few channels)
    (1, 5, 20001, 1e-5, 8, True, False, False),      # five sub-chunks, the last partial
    (2, 3, 12289, 1e-2, 6, True, False, False),      # long channel, early stop: recomputed
    (2, 4, 17000, 1e-5, 6, True, True, True),        # long, warm start held in h, early stop
])
def test_fused_matches_oracle_and_per_iteration(plan, B, D, T, eps, k_max, h0, warm,
                                                in_place):
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=16000 + B * 31 + D * 7 + T + k_max)
    x = I.deer_inputs(w)
    if h0:
        x["h0"] = np.random.default_rng(T).normal(0, 0.5, B * D).astype(np.float32)
    u = x["u"].reshape(B, D, T)
    h_init = None
    if warm:  # near the solution: the sequential loop with u perturbed
        pert = np.random.default_rng(T + 1).normal(0, 0.02, u.shape)
        h_init = oracle.rnn_seq(x["w"], u + pert, x["h0"].reshape(B, D)).astype(np.float32)
    ref_h, ref_it, ref_d = oracle.deer(x["w"], u, x["h0"].reshape(B, D), h_init, eps=eps,
                                       k_max=k_max)
    got = both_paths(plan, x, B, D, T, eps, k_max, h_init, in_place)
    tag = f"deer fused {B}x{D}x{T} eps={eps} k_max={k_max} h0={h0} warm={warm} in_place={in_place}"
    (hf, inf_), (hp, inp) = got["fused"], got["per-iteration"]
    ef, ep, efp = relerr(hf, ref_h), relerr(hp, ref_h), relerr(hf, hp)
    log(f"{tag}: iters fused {inf_['iters']} per-iteration {inp['iters']} oracle {ref_it}; "
        f"deltas {inf_['deltas']} vs {list(ref_d)}; relerr fused {ef:.2e} per-iteration {ep:.2e} "
        f"fused vs per-iteration {efp:.2e}")
    assert inf_["iters"] == inp["iters"] == ref_it
    assert inf_["converged"] == inp["converged"]
    assert ef <= 1e-5 and ep <= 1e-5 and efp <= 1e-5
    assert len(inf_["deltas"]) == len(inp["deltas"])
    for df, dp, do in zip(inf_["deltas"], inp["deltas"], ref_d):
        assert abs(df - do) <= 1e-5 + 1e-3 * do and abs(df - dp) <= 1e-6 + 1e-4 * dp


def test_fused_async_and_repeat(plan):
    """The asynchronous form gives the same iterate and record, and repeated
    solves into the same workspace agree bit for bit."""
    plan(deer_fuse=1)
    B, D, T = 4, 64, 8192
    x = I.deer_inputs(I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=16500))
    w = torch.from_numpy(x["w"]).to(DEV)
    u = torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV)
    h_sync, info = lrs.deer_solve(w, u)
    outs = []
    ws = None
    for _ in range(3):
        h, ws = lrs.deer_solve(w, u, workspace=ws, sync=False)
        outs.append(h)
    torch.cuda.synchronize()
    st = lrs.deer_stats(ws, 5)
    assert st["iters"] == info["iters"] and st["converged"] == info["converged"]
    for h in outs:
        assert torch.equal(h, h_sync)


# SRU whose forget gate reads v_f * c_{t-1}: the fused persistent walk (forced
# with the plan option persist_min_blocks = 0) against the oracle and the per-iteration path.
@pytest.mark.parametrize("B,D,T,io,eps,k_max,warm,in_place", [
    (2, 64, 1000, "bf16", 1e-5, 5, False, False),
    (1, 258, 513, "f32", 1e-5, 8, False, False),     # partial channel block, ragged tiles
    (3, 50, 200, "bf16", 1e-5, 1, False, False),     # K_max = 1
    (2, 64, 777, "f32", 1e-2, 6, False, False),      # early stop: recomputed
    (2, 64, 900, "bf16", 1e-5, 6, True, False),      # warm start
    (2, 64, 900, "f32", 1e-5, 6, True, True),        # warm start held in c_states
])
def test_sru_deer_fused_matches_oracle_and_per_iteration(plan, B, D, T, io, eps, k_max,
                                                          warm, in_place):
    from test_gpu_sru_nl import setup
    plan(persist_min_blocks=0)
    w = I.scaled(I.WORKLOADS["sru_deer"], B=B, D=D, T=T, seed=16800 + B * 13 + D + T + k_max)
    z, z64, p, pd = setup(w, io)
    c0 = np.random.default_rng(T).normal(0, 0.5, (B, D)).astype(np.float32)
    c_init = None
    if warm:  # near the solution: the sequential loop on perturbed pre-activations
        pert = np.random.default_rng(T + 1).normal(0, 0.02, z64["zf"].shape)
        _, c_seq = oracle.sru_nl_seq(z64["zf"] + pert, z64["zr"], z64["zx"], p["bf"], p["br"],
                                     p["vf"], c0)
        c_init = c_seq.astype(np.float32)
    hr, cr, it, dl = oracle.sru_deer(z64["zf"], z64["zr"], z64["zx"], p["bf"], p["br"], p["vf"],
                                     c0=c0, c_init=c_init, eps=eps, k_max=k_max)
    got = {}
    for mode, flag in (("fused", "1"), ("per-iteration", "0")):
        plan(deer_fuse=int(flag))
        ci = None if c_init is None else torch.from_numpy(c_init).to(DEV)
        h, cs, cl, info = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pd["bf"], pd["br"],
                                           pd["vf"], torch.from_numpy(c0).to(DEV), ci, eps=eps,
                                           k_max=k_max, want_c_last=True,
                                           c_states=ci if in_place else None)
        torch.cuda.synchronize()
        got[mode] = (h.float().cpu().numpy(), cs.cpu().numpy(), cl.cpu().numpy(), info)
    (hf, cf, clf, inf_), (hp, cp, clp, inp) = got["fused"], got["per-iteration"]
    e = {"c fused": relerr(cf, cr), "c per-iteration": relerr(cp, cr),
         "c fused vs per-iteration": relerr(cf, cp), "c_last": relerr(clf, cr[-1]),
         "h fused": relerr(hf, hr)}
    log(f"sru-deer fused {io} {B}x{D}x{T} eps={eps} k_max={k_max} warm={warm} in_place={in_place}: "
        f"iters {inf_['iters']} / {inp['iters']} / oracle {it}; "
        + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
    assert inf_["iters"] == inp["iters"] == it
    assert inf_["converged"] == inp["converged"]
    assert e["c fused"] <= 1e-5 and e["c per-iteration"] <= 1e-5
    assert e["c fused vs per-iteration"] <= 1e-5 and e["c_last"] <= 1e-5
    assert e["h fused"] <= (2e-2 if io == "bf16" else 1e-5)


# Per-sequence stopping (lrs_deer_solve_seq) on the fused pass: sequences that
# converge at different speeds, so some stop early (recomputed) and some run
# to K_max; each against the oracle run on that sequence alone and against the
# one-launch-per-iteration path.
@pytest.mark.parametrize("B,D,T,warm,in_place", [(4, 3, 100, False, False),
                                                 (3, 64, 4096, False, False),
                                                 (2, 40, 8000, True, False),
                                                 (4, 8, 6000, True, True),
                                                 (3, 8, 12000, False, False)])
def test_per_sequence_fused(plan, B, D, T, warm, in_place):
    from test_gpu_deer_seq import make
    scales = [0.05, 1.0, 3.0, 0.5][:B]
    w, u, h0 = make(B, D, T, 17000 + T, scales)
    eps, k_max = 1e-5, 8
    h_init = None
    if warm:
        pert = np.random.default_rng(T).normal(0, 0.02, u.shape)
        h_init = oracle.rnn_seq(w, u + pert, h0).astype(np.float32)
    ref = [oracle.deer(w, u[b:b + 1], h0[b:b + 1], None if h_init is None else h_init[b:b + 1],
                       eps=eps, k_max=k_max) for b in range(B)]
    got = {}
    for mode, flag in (("fused", "1"), ("per-iteration", "0")):
        plan(deer_fuse=int(flag))
        hi = None if h_init is None else torch.from_numpy(h_init).to(DEV)
        h, iters, conv = lrs.deer_solve_seq(torch.from_numpy(w).to(DEV),
                                            torch.from_numpy(u).to(DEV),
                                            torch.from_numpy(h0).to(DEV), hi, eps=eps,
                                            k_max=k_max, out=hi if in_place else None)
        torch.cuda.synchronize()
        got[mode] = (h.cpu().numpy(), list(iters), list(conv))
    (hf, itf, cvf), (hp, itp, cvp) = got["fused"], got["per-iteration"]
    log(f"per-sequence fused {B}x{D}x{T} warm={warm} in_place={in_place}: iters fused {itf} "
        f"per-iteration {itp} oracle {[r[1] for r in ref]}")
    assert itf == itp == [r[1] for r in ref]
    assert cvf == cvp
    for b in range(B):
        assert relerr(hf[b:b + 1], ref[b][0]) <= 1e-5
        assert relerr(hf[b:b + 1], hp[b:b + 1]) <= 1e-5


def test_per_sequence_fused_async(plan):
    plan(deer_fuse=1)
    from test_gpu_deer_seq import make
    w, u, h0 = make(3, 16, 3000, 17500, [0.05, 1.0, 3.0])
    wd, ud, h0d = (torch.from_numpy(v).to(DEV) for v in (w, u, h0))
    h_sync, iters, conv = lrs.deer_solve_seq(wd, ud, h0d, k_max=8)
    h_async, ws = lrs.deer_solve_seq(wd, ud, h0d, k_max=8, sync=False)
    torch.cuda.synchronize()
    assert torch.equal(h_sync, h_async)


def test_fused_long_channels_by_default():
    """Channels longer than 8192 steps that number at least the compute units
    take the fused pass under the default options: the same result,
    iteration count and norms as forcing it, against the oracle and the
    one-launch-per-iteration path."""
    B, D, T = 4, 512, 12288
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=16900)
    x = I.deer_inputs(w)
    wd = torch.from_numpy(x["w"]).to(DEV)
    u = torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV)
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    assert B * D >= cus
    h_def, info_def = lrs.deer_solve(wd, u)
    with lrs.plan_options(deer_fuse=1):
        h_f, info_f = lrs.deer_solve(wd, u)
    with lrs.plan_options(deer_fuse=0):
        h_p, info_p = lrs.deer_solve(wd, u)
    torch.cuda.synchronize()
    ref_h, ref_it, ref_d = oracle.deer(x["w"], x["u"].reshape(B, D, T), x["h0"].reshape(B, D),
                                       None, eps=1e-5, k_max=5)
    e = relerr(h_def.cpu().numpy(), ref_h)
    ep = relerr(h_p.cpu().numpy(), ref_h)
    log(f"deer {B}x{D}x{T} default plan: iters {info_def['iters']} (oracle {ref_it}), "
        f"relerr {e:.2e}, per-iteration {ep:.2e}")
    assert torch.equal(h_def, h_f) and info_def == info_f
    assert info_def["iters"] == info_p["iters"] == ref_it
    assert e <= 1e-5 and ep <= 1e-5
