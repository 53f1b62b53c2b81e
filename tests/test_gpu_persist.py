"""The persistent [T,B,D] kernels (one workgroup per channel block walking
all time tiles, chosen when the channel blocks fill the GPU): the SRU forward,
the LSTM forward and the SRU-by-DEER iteration, against the fp64 oracle, forced through
the persist_min_blocks plan option on ragged shapes (partial last tile in time, partial
last channel block, both I/O types, c0, saved cell states and c_T), and at the
full B=32 D=1024 T=2048 shape both ways, where the two kernel families must
agree within the parity bar; with persistence forced, the SRU and SRU-by-DEER
graph replays, the K_max cap, warm starts and the asynchronous form."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, bf16_dev, log
from test_gpu_graph_more import replay_matches
from test_gpu_sru_nl import check as sru_deer_check, run as sru_deer_run

pytestmark = pytest.mark.gpu


def sru_run(w, io, c0=None):
    s = I.sru_inputs(w)
    z64 = {k: I.bf16_bits_to_f64(s[k]) for k in ("zf", "zr", "zx")}
    if io == "bf16":
        z = {k: bf16_dev(s[k]) for k in ("zf", "zr", "zx")}
    else:
        z = {k: torch.from_numpy(z64[k].astype(np.float32)).to(DEV) for k in z64}
    bf, br = (torch.from_numpy(s[k]).to(DEV) for k in ("bias_f", "bias_r"))
    c0d = None if c0 is None else torch.from_numpy(c0).to(DEV)
    cs = torch.empty((w.T, w.B, w.D), dtype=torch.float32, device=DEV)
    h, cl = lrs.sru_fwd(z["zf"], z["zr"], z["zx"], bf, br, c0d, want_c_last=True, c_states=cs)
    torch.cuda.synchronize()
    return h.float().cpu().numpy(), cl.cpu().numpy(), cs.cpu().numpy(), z64, s


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (2, 3, 65), (3, 50, 200), (1, 258, 513),
                                   (2, 128, 1000), (1, 300, 64)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_sru_persistent_ragged(plan, B, D, T, io):
    plan(persist_min_blocks=0)
    w = I.scaled(I.WORKLOADS["sru_fwd"], B=B, D=D, T=T, seed=13000 + B * 7 + D + T)
    c0 = np.random.default_rng(T).normal(size=(B, D)).astype(np.float32)
    h, cl, cs, z64, s = sru_run(w, io, c0)
    ref_h, ref_c = oracle.sru_fwd(z64["zf"], z64["zr"], z64["zx"], s["bias_f"], s["bias_r"], c0)
    e = {"h": relerr(h, ref_h), "c_last": relerr(cl, ref_c), "cs_last_row": relerr(cs[-1], ref_c)}
    log(f"persistent sru {io} {B}x{D}x{T}: " + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
    assert e["h"] <= (2e-2 if io == "bf16" else 1e-5)
    assert e["c_last"] <= 1e-5 and e["cs_last_row"] <= 1e-5


@pytest.mark.parametrize("T", [64, 127, 128, 191, 192, 256, 257, 449])
def test_sru_persistent_tile_counts(plan, T):
    """bf16, B*D a multiple of 8 with a partial last 128-channel block: one to
    seven full tiles of 64 steps, with and without a ragged tail; with saved
    cell states and without them (the walk then computes the same h, bit for
    bit)."""
    plan(persist_min_blocks=0)
    B, D = 2, 132
    w = I.scaled(I.WORKLOADS["sru_fwd"], B=B, D=D, T=T, seed=13100 + T)
    c0 = np.random.default_rng(T + 7).normal(size=(B, D)).astype(np.float32)
    h, cl, cs, z64, s = sru_run(w, "bf16", c0)
    ref_h, ref_c = oracle.sru_fwd(z64["zf"], z64["zr"], z64["zx"], s["bias_f"], s["bias_r"], c0)
    e = {"h": relerr(h, ref_h), "c_last": relerr(cl, ref_c), "cs": relerr(cs[-1], ref_c)}
    z = {k: bf16_dev(s[k]) for k in ("zf", "zr", "zx")}
    bf, br = (torch.from_numpy(s[k]).to(DEV) for k in ("bias_f", "bias_r"))
    h2 = lrs.sru_fwd(z["zf"], z["zr"], z["zx"], bf, br, torch.from_numpy(c0).to(DEV))
    torch.cuda.synchronize()
    log(f"persistent sru bf16 {B}x{D}x{T}: " + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
    assert e["h"] <= 2e-2 and e["c_last"] <= 1e-5 and e["cs"] <= 1e-5
    assert np.array_equal(h2.float().cpu().numpy(), h)


def test_sru_both_kernels_at_workload_shape(plan):
    w = I.WORKLOADS["sru_fwd"]
    outs = {}
    for mode, lim in (("persistent", 0), ("tiles", 1 << 40)):
        plan(persist_min_blocks=lim)
        outs[mode] = sru_run(w, "bf16")[:3]
    s = I.sru_inputs(w)
    ref_h, ref_c = oracle.sru_fwd(*(I.bf16_bits_to_f64(s[k]) for k in ("zf", "zr", "zx")),
                                  s["bias_f"], s["bias_r"])
    for mode, (h, cl, cs) in outs.items():
        eh, ec = relerr(h, ref_h), relerr(cl, ref_c)
        log(f"sru_fwd workload, {mode}: h={eh:.2e} c_last={ec:.2e}")
        assert eh <= 2e-2 and ec <= 1e-5
    # the saved cell states of the two kernel families agree (fp32 bar)
    assert relerr(outs["persistent"][2], outs["tiles"][2]) <= 1e-5


@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (1, 3, 7), (2, 5, 64), (3, 50, 200),
                                   (1, 258, 513), (2, 128, 1000)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_sru_deer_persistent_ragged(plan, B, D, T, io):
    plan(persist_min_blocks=0)
    w = I.scaled(I.WORKLOADS["sru_deer"], B=B, D=D, T=T, seed=13200 + B * 13 + D * 5 + T)
    c0 = np.random.default_rng(T + D + 1).normal(size=(B, D)).astype(np.float32)
    sru_deer_check(*sru_deer_run(w, io, c0=c0, k_max=8), io, f"persistent sru-deer {io} {B}x{D}x{T}")


def test_sru_deer_both_kernels_at_workload_shape(plan):
    w = I.WORKLOADS["sru_deer"]
    for mode, lim in (("persistent", 0), ("tiles", 1 << 40)):
        plan(persist_min_blocks=lim)
        sru_deer_check(*sru_deer_run(w, "bf16"), "bf16", f"sru_deer workload, {mode}")


def test_sru_deer_persistent_graph(plan):
    plan(persist_min_blocks=0)
    w = I.scaled(I.WORKLOADS["sru_deer"], B=2, D=128, T=1000, seed=13300)
    s = I.sru_inputs(w)
    z = {k: bf16_dev(s[k]) for k in ("zf", "zr", "zx")}
    bf, br = (torch.from_numpy(s[k]).to(DEV) for k in ("bias_f", "bias_r"))
    vf = torch.from_numpy(I.sru_vf(w)).to(DEV)
    h = torch.empty_like(z["zf"])
    cs = torch.empty((1000, 2, 128), device=DEV)
    ws = torch.empty(lrs.load().lrs_sru_deer_workspace_bytes(1000, 2, 128, 5), dtype=torch.uint8,
                     device=DEV)

    def step():
        lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], bf, br, vf, out=h, c_states=cs, workspace=ws,
                         sync=False)
    replay_matches(step, [h, cs], False, "persistent sru deer")


@pytest.mark.parametrize("name", ["test_sru_graph_replay", "test_sru_fwd_bwd_graph_replay"])
def test_sru_persistent_graph(plan, name):
    """The SRU graph replays (alone, and with the backward in the same graph)
    with the persistent forward forced."""
    import test_gpu_graph
    plan(persist_min_blocks=0)
    getattr(test_gpu_graph, name)()


@pytest.mark.parametrize("name", ["test_kmax_cap_and_warm_start", "test_async_form_and_stats",
                                  "test_linear_case_matches_sru_layer"])
def test_sru_deer_persistent_options(plan, name):
    """The K_max cap, warm starts in place, the asynchronous form and the
    v_f = 0 case with the persistent iteration forced."""
    import test_gpu_sru_nl
    plan(persist_min_blocks=0)
    getattr(test_gpu_sru_nl, name)()


# LSTM cell-state layer: the persistent forward (chosen at the workload shape,
# forced here on ragged shapes) against the oracle, the backward fed its saved
# cell states, and both forward kernel families at the workload shape.
@pytest.mark.parametrize("B,D,T", [(1, 1, 1), (2, 3, 65), (3, 50, 200), (1, 258, 513),
                                   (2, 128, 1000), (1, 300, 64)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_lstm_persistent_ragged(plan, B, D, T, io):
    from test_gpu_lstm import check, run_case
    plan(persist_min_blocks=0)
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=B, D=D, T=T, seed=13500 + B * 11 + D * 3 + T)
    rng = np.random.default_rng(T + 7 * D)
    c0 = rng.normal(size=(B, D)).astype(np.float32)
    gcl = rng.normal(size=(B, D)).astype(np.float32)
    check(run_case(w, io, c0=c0, gcl=gcl), io, f"persistent lstm {io} {B}x{D}x{T}")


def test_lstm_both_kernels_at_workload_shape(plan):
    from test_gpu_lstm import dev_inputs
    w = I.WORKLOADS["lstm_fwd_bwd"]
    z, z64 = dev_inputs(w, "bf16")
    outs = {}
    for mode, lim in (("persistent", 0), ("tiles", 1 << 40)):
        plan(persist_min_blocks=lim)
        cs = torch.empty((w.T, w.B, w.D), dtype=torch.float32, device=DEV)
        h, cl = lrs.lstm_fwd(z["zf"], z["zi"], z["zc"], z["zo"], want_c_last=True, c_states=cs)
        torch.cuda.synchronize()
        outs[mode] = (h.float().cpu().numpy(), cl.cpu().numpy(), cs.cpu().numpy())
    ref_h, ref_c = oracle.lstm_fwd(*(z64[k] for k in ("zf", "zi", "zc", "zo")))
    for mode, (h, cl, cs) in outs.items():
        eh, ec = relerr(h, ref_h), relerr(cl, ref_c)
        log(f"lstm_fwd workload, {mode}: h={eh:.2e} c_last={ec:.2e}")
        assert eh <= 2e-2 and ec <= 1e-5
        assert relerr(cs[-1], ref_c) <= 1e-5
    assert relerr(outs["persistent"][2], outs["tiles"][2]) <= 1e-5


def test_lstm_persistent_graph(plan):
    """The LSTM forward + backward graph replays with the persistent forward."""
    import test_gpu_graph_more
    plan(persist_min_blocks=0)
    test_gpu_graph_more.test_lstm_graph()
