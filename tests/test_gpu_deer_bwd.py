"""Backward of the nonlinear RNN at its solution (lrs_deer_bwd) against the
fp64 oracle on identical inputs: ragged, single- and multi-chunk shapes with
the sequential solution as h, and the DEER shape with the GPU solve's own
result as h.  Bar: 1e-5 (fp32 I/O) for dL/du, dL/dw and dL/dh0."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def grads_vs_oracle(x, h32, g32, B, D, T, tag):
    h0 = x["h0"].reshape(B, D).astype(np.float32)
    gu, gw, gh0 = lrs.deer_bwd(torch.from_numpy(x["w"]).to(DEV),
                               torch.from_numpy(h32).to(DEV), torch.from_numpy(g32).to(DEV),
                               torch.from_numpy(h0).to(DEV))
    torch.cuda.synchronize()
    ru, rw, rh0 = oracle.deer_bwd(x["w"], h32, g32, h0)
    errs = {"du": relerr(gu.cpu().numpy(), ru), "dw": relerr(gw.cpu().numpy(), rw),
            "dh0": relerr(gh0.cpu().numpy(), rh0)}
    log(f"{tag}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= 1e-5, (k, e)


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (1, 3, 7), (2, 5, 1000), (1, 4, 4096),
                                   (1, 3, 4097), (2, 2, 30001), (1, 2, 70000)])
def test_deer_bwd_ragged(B, D, T):
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=8000 + T)
    x = I.deer_inputs(w)
    h = oracle.rnn_seq(x["w"], x["u"].reshape(B, D, T), x["h0"].reshape(B, D)).astype(np.float32)
    g = I.series(w.seed, "g", ("normal", 0.0, 1.0), np.arange(w.C), T,
                 np.float32).reshape(B, D, T)
    grads_vs_oracle(x, h, g, B, D, T, f"deer bwd B={B} D={D} T={T}")


def test_deer_solve_then_bwd_workload():
    """B=16 D=512 T=8192: solve on the GPU, then the backward at that solution."""
    w = I.WORKLOADS["deer"]
    B, D, T = w.B, w.D, w.T
    x = I.deer_inputs(w)
    u = torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV)
    h, info = lrs.deer_solve(torch.from_numpy(x["w"]).to(DEV), u,
                             torch.from_numpy(x["h0"].reshape(B, D)).to(DEV))
    g = I.series(w.seed, "g", ("normal", 0.0, 1.0), np.arange(w.C), T,
                 np.float32).reshape(B, D, T)
    grads_vs_oracle(x, h.cpu().numpy(), g, B, D, T, f"deer solve+bwd iters={info['iters']}")


def test_deer_bwd_deterministic():
    B, D, T = 3, 40, 9000
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=8100)
    x = I.deer_inputs(w)
    h = torch.from_numpy(oracle.rnn_seq(x["w"], x["u"].reshape(B, D, T)).astype(np.float32)).to(DEV)
    g = torch.randn(B, D, T, device=DEV)
    wd = torch.from_numpy(x["w"]).to(DEV)
    a = lrs.deer_bwd(wd, h, g)[1].clone()
    b = lrs.deer_bwd(wd, h, g)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
