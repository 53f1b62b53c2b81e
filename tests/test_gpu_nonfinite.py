"""A NaN in one element of a DEER input must surface as a non-finite update in
every solve path: the fused pass with 4 and with 8 steps per lane, the
one-launch-per-iteration path for long channels, the per-sequence stop rule
(only the sequence holding the NaN is affected) and SRU-by-DEER through both
its tile iteration and its fused persistent walk.  The update norm is folded
with a NaN-propagating maximum, so the NaN must win over every finite update
and the solve must run to K_max and report LRS_ERR_NONFINITE (not converged).
A clean solve of the same inputs is run first as the control."""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import binding
from linear_recurrence_scan_diagonal_amd import inputs as I
from gpu_util import DEV, bf16_dev, log

pytestmark = pytest.mark.gpu
NONFINITE = binding.LRS_ERR_NONFINITE


def deer_tensors(B, D, T, seed):
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=seed)
    x = I.deer_inputs(w)
    return (torch.from_numpy(x["w"]).to(DEV),
            torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV))


# T = 500: fused pass, 4 steps per lane; T = 8192: fused pass, 8 steps per
# lane over two 4096-step sub-chunks; T = 30001: one launch per iteration.
@pytest.mark.parametrize("T", [500, 8192, 30001])
def test_deer_nan_is_nonfinite(T):
    B, D, k_max = 2, 4, 8
    wd, u = deer_tensors(B, D, T, 14000 + T)
    _, clean = lrs.deer_solve(wd, u, k_max=k_max)
    torch.cuda.synchronize()
    assert clean["status"] == binding.LRS_OK and clean["converged"], clean
    u[1, 2, (2 * T) // 3] = float("nan")
    h, info = lrs.deer_solve(wd, u, k_max=k_max)
    torch.cuda.synchronize()
    log(f"deer T={T}: clean {clean['iters']} iterations; with a NaN {info}")
    assert info["status"] == NONFINITE
    assert not info["converged"] and info["iters"] == k_max
    assert np.isnan(info["deltas"][-1])
    assert torch.isnan(h[1, 2]).any()
    assert torch.isfinite(h[0]).all()  # other channels are untouched by the NaN


@pytest.mark.parametrize("T", [500, 8192])
def test_deer_seq_nan_stays_in_its_sequence(T):
    B, D, k_max = 3, 4, 8
    wd, u = deer_tensors(B, D, T, 14100 + T)
    _, it0, conv0 = lrs.deer_solve_seq(wd, u, k_max=k_max)
    torch.cuda.synchronize()
    assert all(conv0), (it0, conv0)
    u[1, 0, T // 5] = float("nan")
    _, it, conv = lrs.deer_solve_seq(wd, u, k_max=k_max)
    torch.cuda.synchronize()
    log(f"deer per-sequence T={T}: clean {it0}; sequence 1 with a NaN {it} {conv}")
    assert conv == [True, False, True]
    assert it[1] == k_max
    assert it[0] == it0[0] and it[2] == it0[2]


@pytest.mark.parametrize("persist", [False, True])
def test_sru_deer_nan_is_nonfinite(plan, persist):
    plan(persist_min_blocks=0 if persist else 1 << 40)
    B, D, T, k_max = 2, 128, 300, 8
    w = I.scaled(I.WORKLOADS["sru_deer"], B=B, D=D, T=T, seed=14200)
    s = I.sru_inputs(w)
    z = {k: bf16_dev(s[k]) for k in ("zf", "zr", "zx")}
    bf, br = (torch.from_numpy(s[k]).to(DEV) for k in ("bias_f", "bias_r"))
    vf = torch.from_numpy(I.sru_vf(w)).to(DEV)
    _, _, _, clean = lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], bf, br, vf, k_max=k_max)
    torch.cuda.synchronize()
    assert clean["status"] == binding.LRS_OK and clean["converged"], clean
    zx = z["zx"].clone()
    zx[T // 2, 1, 77] = float("nan")
    h, cs, _, info = lrs.sru_deer_fwd(z["zf"], z["zr"], zx, bf, br, vf, k_max=k_max)
    torch.cuda.synchronize()
    log(f"sru-deer persist={persist}: clean {clean['iters']} iterations; with a NaN {info}")
    assert info["status"] == NONFINITE
    assert not info["converged"] and info["iters"] == k_max
    assert torch.isnan(cs[T // 2:, 1, 77]).all()
    assert torch.isfinite(cs[:, 0]).all()
