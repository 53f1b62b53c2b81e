"""More entry points captured in a HIP graph: the fused forward + backward
scan, the packed short-channel scans, the LSTM layer forward + backward, the
asynchronous SRU-by-DEER solve, the asynchronous DEER solve with
per-sequence stopping and the sequential tanh RNN (both buffer-resource forms:
T % 4 == 0 and not).  Every replay (interleaved with unrelated eager work
and host synchronisations, outputs poisoned with NaN before each) must
reproduce the eager run: bit for bit where the association order is fixed,
else within the parity bar (1e-5)."""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, bf16_dev, log, to_dev

pytestmark = pytest.mark.gpu


def replay_matches(step, outs, exact, tag):
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    a = torch.rand(1000, device=DEV)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        (a * 2.0).sum().item()  # unrelated eager work and a host synchronisation
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            if exact:
                assert torch.equal(o, r), (tag, rep, i)
            else:
                assert relerr(o.float().cpu().numpy(), r.float().cpu().numpy()) <= 1e-5, (tag, rep, i)
    log(f"{tag}: 4 replays match")


def scan_tensors(B, D, T, seed):
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=seed)
    x = I.scan_inputs(w)
    t = {k: to_dev(x[k], B, D, T, "bdt") for k in ("a", "b", "g")}
    t["h0"] = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    return t


def test_fused_scan_graph():
    t = scan_tensors(2, 64, 4096, 12000)
    out = (torch.empty_like(t["a"]), torch.empty_like(t["a"]), torch.empty_like(t["a"]),
           torch.empty((2, 64), device=DEV))
    replay_matches(lambda: lrs.scan_fwd_bwd(t["a"], t["b"], t["g"], t["h0"], out=out), out, True,
                   "fused scan")


@pytest.mark.parametrize("T", [3, 32])
def test_short_scan_graph(T):
    t = scan_tensors(4, 300, T, 12100 + T)
    h = torch.empty_like(t["a"])
    ga, gb = torch.empty_like(t["a"]), torch.empty_like(t["a"])
    gh0 = torch.empty((4, 300), device=DEV)

    def step():
        lrs.scan_fwd(t["a"], t["b"], t["h0"], out=h)
        lrs.scan_bwd(t["a"], h, t["g"], t["h0"], grad_a=ga, grad_b=gb, grad_h0=gh0)
    replay_matches(step, [h, ga, gb, gh0], True, f"short scan T={T}")


def test_lstm_graph():
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=4, D=256, T=600, seed=12200)
    s = I.lstm_inputs(w)
    s["gh"] = I.sru_grad_inputs(w)["gh"]
    z = {k: bf16_dev(v) for k, v in s.items()}
    gates = (z["zf"], z["zi"], z["zc"], z["zo"])
    h = torch.empty_like(z["zf"])
    cs = torch.empty((600, 4, 256), device=DEV)
    grads = tuple(torch.empty_like(z["zf"]) for _ in range(4)) + (torch.empty((4, 256), device=DEV),)
    ws = torch.empty(max(1, lrs.load().lrs_lstm_workspace_bytes(600, 4, 256)), dtype=torch.uint8,
                     device=DEV)

    def step():
        lrs.lstm_fwd(*gates, out=h, c_states=cs, workspace=ws)
        lrs.lstm_bwd(*gates, cs, z["gh"], out=grads, workspace=ws)
    replay_matches(step, [h, cs, *grads], False, "lstm")


def test_sru_deer_graph():
    w = I.scaled(I.WORKLOADS["sru_deer"], B=2, D=128, T=1000, seed=12300)
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
    replay_matches(step, [h, cs], False, "sru deer")


def test_deer_seq_graph():
    w = I.scaled(I.WORKLOADS["deer"], B=3, D=16, T=3000, seed=12400)
    x = I.deer_inputs(w)
    u = x["u"].reshape(3, 16, 3000) * np.array([0.1, 1.0, 2.0], dtype=np.float32)[:, None, None]
    wd, ud = torch.from_numpy(x["w"]).to(DEV), torch.from_numpy(u.astype(np.float32)).to(DEV)
    h = torch.empty_like(ud)
    ws = torch.empty(lrs.load().lrs_deer_seq_workspace_bytes(3, 16, 3000, 5), dtype=torch.uint8,
                     device=DEV)
    replay_matches(lambda: lrs.deer_solve_seq(wd, ud, out=h, workspace=ws, sync=False), [h], True,
                   "deer per-sequence")


@pytest.mark.parametrize("layout,B,D,T", [("bdt", 2, 3, 20000), ("bdt", 4, 8, 300),
                                          ("tbd", 2, 70, 3000)])
def test_bf16_scan_graph(layout, B, D, T):
    """The scan pair and the one-call forward + backward with bf16 arrays,
    captured once and replayed: look-back chunks ([B,D,T], 20000 steps),
    single-chunk channels and [T,B,D] time blocks; every replay bit for bit
    the eager result (the carry order is fixed)."""
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd_bf16"], B=B, D=D, T=T, seed=19500 + T)
    x = I.scan_inputs_bf16(w)
    a, b, g = (to_dev(x[k].view(np.int16), B, D, T, layout).view(torch.bfloat16)
               for k in ("a", "b", "g"))
    h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(DEV)
    h, ga, gb = (torch.empty_like(a) for _ in range(3))
    gh0 = torch.empty((B, D), device=DEV)
    ws = torch.empty(lrs.scan_workspace_bytes(B, D, T, layout, torch.bfloat16) + 4096,
                     dtype=torch.uint8, device=DEV)

    def step():
        lrs.scan_fwd(a, b, h0, layout=layout, out=h, workspace=ws)
        lrs.scan_bwd(a, h, g, h0, layout=layout, grad_a=ga, grad_b=gb, grad_h0=gh0, workspace=ws)
    replay_matches(step, (h, ga, gb, gh0), exact=True, tag=f"bf16 scan graph {layout} {B}x{D}x{T}")
    if layout == "bdt":
        out = tuple(torch.empty_like(t) for t in (h, ga, gb, gh0))

        def fused():
            lrs.scan_fwd_bwd(a, b, g, h0, out=out, workspace=ws)
        replay_matches(fused, out, exact=True, tag=f"bf16 fused scan graph {B}x{D}x{T}")


@pytest.mark.parametrize("T", [4096, 1001])
def test_rnn_seq_graph(T):
    B, D = 2, 100
    x = I.deer_inputs(I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=12900 + T))
    w = torch.from_numpy(x["w"]).to(DEV)
    u = torch.from_numpy(x["u"].reshape(B, D, T)).to(DEV)
    h0 = torch.from_numpy(np.full((B, D), 0.25, np.float32)).to(DEV)
    out = (torch.empty_like(u),)
    replay_matches(lambda: lrs.rnn_seq(w, u, h0, out=out[0]), out, True, f"rnn_seq T={T}")
