"""DEER with per-sequence stopping on the GPU (lrs_deer_solve_seq) against the
fp64 oracle run on each sequence alone: per-sequence iteration counts equal,
every sequence's result within the fp32 bar 1e-5.  Sequences are made to
converge at different speeds by scaling u per batch entry; shapes cover one
workgroup per channel, two sub-chunks and the multi-chunk look-back."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def make(B, D, T, seed, scales):
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=seed)
    x = I.deer_inputs(w)
    u = x["u"].reshape(B, D, T) * np.asarray(scales, dtype=np.float32)[:, None, None]
    h0 = np.random.default_rng(seed).normal(0, 0.5, size=(B, D)).astype(np.float32)
    return x["w"], u.astype(np.float32), h0


@pytest.mark.parametrize("B,D,T", [(4, 3, 100), (3, 64, 4096), (2, 40, 8000), (3, 5, 20000)])
def test_per_sequence_counts_and_results(B, D, T):
    scales = [0.05, 1.0, 3.0, 0.5][:B]
    w, u, h0 = make(B, D, T, 11000 + T, scales)
    eps, k_max = 1e-5, 12
    h, iters, conv = lrs.deer_solve_seq(torch.from_numpy(w).to(DEV), torch.from_numpy(u).to(DEV),
                                        torch.from_numpy(h0).to(DEV), eps=eps, k_max=k_max)
    torch.cuda.synchronize()
    hg = h.cpu().numpy()
    ref_iters = []
    for b in range(B):
        hr, it, dl = oracle.deer(w, u[b:b + 1], h0[b:b + 1], eps=eps, k_max=k_max)
        ref_iters.append(it)
        e = relerr(hg[b:b + 1], hr)
        log(f"seq {b} scale {scales[b]}: iters {iters[b]} vs {it} (deltas {list(dl)}), relerr {e:.2e}")
        assert iters[b] == it
        assert conv[b] == (dl[-1] < eps)
        assert e <= 1e-5
    assert len(set(ref_iters)) > 1, "sequences should converge at different iterations"


def test_async_matches_sync():
    w, u, h0 = make(3, 32, 3000, 11100, [0.1, 1.0, 2.0])
    wd, ud, h0d = (torch.from_numpy(v).to(DEV) for v in (w, u, h0))
    h1, it1, _ = lrs.deer_solve_seq(wd, ud, h0d)
    h2, ws = lrs.deer_solve_seq(wd, ud, h0d, sync=False)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)


def test_uniform_sequences_match_global_solve(plan):
    """When every sequence needs the same iterations the result is the global
    solve's: bit for bit between like paths (fused pass against fused pass,
    one launch per iteration against the same), and within the parity bar
    between the two paths (same iterations, another rounding order at wave
    edges)."""
    w, u, h0 = make(2, 16, 2048, 11200, [1.0, 1.0])
    wd, ud, h0d = (torch.from_numpy(v).to(DEV) for v in (w, u, h0))
    hs_f, its_f, _ = lrs.deer_solve_seq(wd, ud, h0d, k_max=8)
    hg_f, info_f = lrs.deer_solve(wd, ud, h0d, k_max=8)
    plan(deer_fuse=0)
    hs_u, its_u, _ = lrs.deer_solve_seq(wd, ud, h0d, k_max=8)
    hg_u, info_u = lrs.deer_solve(wd, ud, h0d, k_max=8)
    torch.cuda.synchronize()
    itg = info_u["iters"]
    log(f"per-sequence fused {its_f} / per-iteration {its_u}, global fused {info_f['iters']} / "
        f"per-iteration {itg}")
    assert list(its_f) == list(its_u)
    assert info_f["iters"] == itg
    assert relerr(hg_f.cpu().numpy(), hg_u.cpu().numpy()) <= 1e-5
    if len(set(its_u)) == 1 and its_u[0] == itg:
        assert torch.equal(hs_f, hg_f)
        assert torch.equal(hs_u, hg_u)
    else:
        assert max(its_u) == itg
