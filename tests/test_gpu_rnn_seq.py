"""The sequential tanh RNN (lrs_rnn_seq: h_t = tanh(w h_{t-1} + u_t) one step
after another, one lane per channel), the reference point for the DEER solve,
against the oracle's sequential fp64 loop on identical inputs: ragged channel
counts and lengths (partial waves, partial 64-step tiles), a starting state,
saturating inputs, and the DEER workload in full, where it must also agree with
the solve's result.  Bar: 1e-5 (fp32 I/O)."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def run(B, D, T, seed, with_h0, u_scale=1.0):
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=seed)
    x = I.deer_inputs(w)
    u = (x["u"] * np.float32(u_scale)).astype(np.float32).reshape(B, D, T)
    h0 = (I.to_f32(I.params(seed, "h0", ("uniform", -1.0, 1.0), (B * D,))).reshape(B, D)
          if with_h0 else None)
    h = lrs.rnn_seq(torch.from_numpy(x["w"]).to(DEV), torch.from_numpy(u).to(DEV),
                    None if h0 is None else torch.from_numpy(h0).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.rnn_seq(x["w"], u, h0)
    return h, ref, x, u, h0


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (2, 3, 5), (1, 64, 64), (1, 65, 65), (2, 70, 300),
                                   (3, 5, 129), (1, 2, 20000)])
@pytest.mark.parametrize("with_h0", [False, True])
def test_rnn_seq_matches_oracle(B, D, T, with_h0):
    h, ref, *_ = run(B, D, T, 26000 + 7 * T + D, with_h0)
    e = relerr(h.double().cpu().numpy(), ref)
    log(f"rnn_seq B={B} D={D} T={T} h0={with_h0}: {e:.2e}")
    assert e <= 1e-5


def test_rnn_seq_saturating_inputs():
    # |u| up to about 200: tanh saturates to +-1 exactly on most steps
    h, ref, *_ = run(2, 33, 500, 26100, True, u_scale=50.0)
    hn = h.double().cpu().numpy()
    e = relerr(hn, ref)
    log(f"rnn_seq saturating: {e:.2e}, |h| max {np.abs(hn).max()}")
    assert e <= 1e-5 and np.abs(hn).max() <= 1.0


def test_rnn_seq_deer_workload_and_solve():
    w = I.WORKLOADS["deer"]
    B, D, T = w.B, w.D, w.T
    h, ref, x, u, _ = run(B, D, T, w.seed, False)
    e = relerr(h.double().cpu().numpy(), ref)
    hd, info = lrs.deer_solve(torch.from_numpy(x["w"]).to(DEV), torch.from_numpy(u).to(DEV))
    torch.cuda.synchronize()
    es = relerr(h.double().cpu().numpy(), hd.double().cpu().numpy())
    log(f"rnn_seq deer workload B={B} D={D} T={T}: vs oracle {e:.2e}, vs the DEER solve "
        f"({info['iters']} iterations) {es:.2e}")
    assert e <= 1e-5 and es <= 1e-5
