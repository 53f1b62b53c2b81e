"""Randomised parity: every entry point on shapes, seeds and options drawn by
hypothesis (derandomised, so every run draws the same cases), against the
fp64 oracle to the same bars as the fixed-shape tests.  The shape strategies
mix short channels (packed and sequential kernels), channels of one workgroup
and channels spanning several look-back chunks, channel counts that are not
multiples of the tile width, both layouts, both I/O types and optional
arguments present or absent."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, assume, given, settings, strategies as st

import oracle
import linear_recurrence_scan_diagonal_amd as lrs
from linear_recurrence_scan_diagonal_amd import inputs as I
from conftest import relerr
from gpu_util import DEV, from_dev, log, to_dev
from test_gpu_deer_bwd import grads_vs_oracle
from test_gpu_lstm import check as lstm_check, run_case as lstm_case
from test_gpu_scan import compare, oracle_scan, run_scan
from test_gpu_scan_fused import run_fused
from test_gpu_sru_bwd import check as sru_bwd_check, sru_bwd_case
from test_gpu_sru_nl import check as sru_nl_check, run as sru_nl_run

pytestmark = pytest.mark.gpu

MAX_ELEMS = 1 << 21  # keeps each oracle call well under a second


def cases(n):
    return settings(max_examples=n, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))


steps = st.one_of(st.integers(1, 70), st.integers(70, 9000), st.integers(9000, 40000))
layer_steps = st.one_of(st.integers(1, 40), st.integers(40, 3000))
seeds = st.integers(0, 2 ** 31 - 1)


@cases(40)
@given(B=st.integers(1, 4), D=st.integers(1, 300), T=steps, layout=st.sampled_from(["bdt", "tbd"]),
       h0=st.booleans(), seed=seeds)
def test_scan_random(B, D, T, layout, h0, seed):
    assume(B * D * T <= MAX_ELEMS)
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=seed)
    x = I.scan_inputs(w)
    compare(run_scan(x, B, D, T, layout, h0=h0), oracle_scan(x, h0=h0),
            tag=f"random scan {layout} {B}x{D}x{T} h0={h0} seed={seed}")


@cases(30)
@given(B=st.integers(1, 4), D=st.integers(1, 300), T=steps, layout=st.sampled_from(["bdt", "tbd"]),
       h0=st.booleans(), fused=st.booleans(), seed=seeds)
def test_scan_bf16_random(B, D, T, layout, h0, fused, seed):
    """bf16 arrays: the scan pair (or, in [B,D,T], the one-call form); the
    backward against the oracle fed the bf16 h the GPU stored."""
    assume(B * D * T <= MAX_ELEMS)
    if fused:
        assume(layout == "bdt")
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd_bf16"], B=B, D=D, T=T, seed=seed)
    x = I.scan_inputs_bf16(w)
    C = B * D
    dev = {k: to_dev(x[k].view(np.int16), B, D, T, layout).view(torch.bfloat16) for k in ("a", "b", "g")}
    h0v = x["h0"].astype(np.float32) if h0 else np.zeros(C, np.float32)
    h0d = torch.from_numpy(h0v.reshape(B, D)).to(DEV) if h0 else None
    if fused:
        h, da, db, dh0 = lrs.scan_fwd_bwd(dev["a"], dev["b"], dev["g"], h0d)
    else:
        h = lrs.scan_fwd(dev["a"], dev["b"], h0d, layout=layout)
        da, db, dh0 = lrs.scan_bwd(dev["a"], h, dev["g"], h0d, layout=layout)
    torch.cuda.synchronize()
    f64 = {k: I.bf16_bits_to_f64(x[k]) for k in ("a", "b", "g")}
    back = lambda t: I.bf16_bits_to_f64(from_dev(t.view(torch.int16), B, D, T, layout).view(np.uint16))
    h64 = back(h)
    ref_h = oracle.scan_fwd(f64["a"], f64["b"], h0v.astype(np.float64))
    # the one-call form keeps h in fp32 between its passes when a channel fits one kernel
    h_used = ref_h if (fused and T <= 8192) else h64
    ref_da, ref_db, ref_dh0 = oracle.scan_bwd(f64["a"], h_used, h0v.astype(np.float64), f64["g"])
    e = {"h": relerr(h64, ref_h), "da": relerr(back(da), ref_da), "db": relerr(back(db), ref_db),
         "dh0": relerr(dh0.cpu().numpy().reshape(-1).astype(np.float64), ref_dh0)}
    tag = f"random bf16 scan {layout} {B}x{D}x{T} h0={h0} fused={fused} seed={seed}"
    log(tag + ": " + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))
    assert e["h"] <= 2e-2 and e["da"] <= 2e-2 and e["db"] <= 2e-2 and e["dh0"] <= 1e-5, tag


@cases(25)
@given(B=st.integers(1, 4), D=st.integers(1, 200), T=steps, want_h=st.booleans(), seed=seeds)
def test_scan_fwd_bwd_random(B, D, T, want_h, seed):
    assume(B * D * T <= MAX_ELEMS)
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd"], B=B, D=D, T=T, seed=seed)
    x = I.scan_inputs(w)
    if not want_h:  # the one-kernel form only; longer channels need h between the passes
        assume(T <= 8192)
    ref = oracle_scan(x)
    if not want_h:
        del ref["h"]
    compare(run_fused(x, B, D, T, want_h=want_h), ref,
            tag=f"random fused {B}x{D}x{T} want_h={want_h} seed={seed}")


@cases(25)
@given(B=st.integers(1, 3), D=st.integers(1, 300), T=layer_steps,
       io=st.sampled_from(["bf16", "f32"]), c0=st.booleans(), gcl=st.booleans(), seed=seeds)
def test_sru_fwd_bwd_random(B, D, T, io, c0, gcl, seed):
    assume(B * D * T <= MAX_ELEMS)
    w = I.scaled(I.WORKLOADS["sru_fwd_bwd"], B=B, D=D, T=T, seed=seed)
    rng = np.random.default_rng(seed)
    c0v = rng.normal(size=(B, D)).astype(np.float32) if c0 else None
    gclv = rng.normal(size=(B, D)).astype(np.float32) if gcl else None
    got, ref = sru_bwd_case(w, io, c0v, gclv)
    sru_bwd_check(got, ref, io, f"random sru fwd+bwd {io} {B}x{D}x{T} seed={seed}")


@cases(20)
@given(B=st.integers(1, 3), D=st.integers(1, 300), T=layer_steps,
       io=st.sampled_from(["bf16", "f32"]), c0=st.booleans(), seed=seeds)
def test_lstm_random(B, D, T, io, c0, seed):
    assume(B * D * T <= MAX_ELEMS)
    w = I.scaled(I.WORKLOADS["lstm_fwd_bwd"], B=B, D=D, T=T, seed=seed)
    rng = np.random.default_rng(seed)
    c0v = rng.normal(size=(B, D)).astype(np.float32) if c0 else None
    gclv = rng.normal(size=(B, D)).astype(np.float32) if c0 else None
    lstm_check(lstm_case(w, io, c0v, gclv), io, f"random lstm {io} {B}x{D}x{T} seed={seed}")


def robust_count(deltas, eps):
    """True when no norm lies within a factor 2 of eps, so fp32 and fp64 runs
    must stop after the same number of iterations."""
    return all(not (eps / 2 <= d <= 2 * eps) for d in deltas)


@cases(25)
@given(B=st.integers(1, 4), D=st.integers(1, 300), T=steps, h0=st.booleans(), seed=seeds)
def test_rnn_seq_random(B, D, T, h0, seed):
    assume(B * D * T <= MAX_ELEMS)
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=seed)
    x = I.deer_inputs(w)
    u = x["u"].reshape(B, D, T)
    hz = (np.random.default_rng(seed).uniform(-1, 1, (B, D)).astype(np.float32) if h0
          else None)
    h = lrs.rnn_seq(torch.from_numpy(x["w"]).to(DEV), torch.from_numpy(u).to(DEV),
                    None if hz is None else torch.from_numpy(hz).to(DEV))
    torch.cuda.synchronize()
    e = relerr(h.cpu().numpy(), oracle.rnn_seq(x["w"], u, hz))
    log(f"random rnn_seq {B}x{D}x{T} h0={h0} seed={seed}: {e:.2e}")
    assert e <= 1e-5


@cases(25)
@given(B=st.integers(1, 4), D=st.integers(1, 100), T=steps, k_max=st.integers(1, 8),
       eps=st.sampled_from([1e-3, 1e-5, 1e-6]), warm=st.booleans(), seed=seeds)
def test_deer_random(B, D, T, k_max, eps, warm, seed):
    assume(B * D * T <= MAX_ELEMS // 2)
    w = I.scaled(I.WORKLOADS["deer"], B=B, D=D, T=T, seed=seed)
    x = I.deer_inputs(w)
    u = x["u"].reshape(B, D, T)
    h0 = x["h0"].reshape(B, D)
    h_init = None
    if warm:  # a warm start near the solution: the sequential loop with u perturbed
        pert = np.random.default_rng(seed).normal(0, 0.05, u.shape)
        h_init = oracle.rnn_seq(x["w"], u + pert, h0).astype(np.float32)
    ref_h, ref_it, ref_d = oracle.deer(x["w"], u, h0, h_init, eps=eps, k_max=k_max)
    assume(robust_count(ref_d, eps))
    hid = None if h_init is None else torch.from_numpy(h_init).to(DEV)
    h, info = lrs.deer_solve(torch.from_numpy(x["w"]).to(DEV), torch.from_numpy(u).to(DEV),
                             torch.from_numpy(h0).to(DEV), hid, eps=eps, k_max=k_max)
    torch.cuda.synchronize()
    e = relerr(h.cpu().numpy(), ref_h)
    log(f"random deer {B}x{D}x{T} k_max={k_max} eps={eps} warm={warm} seed={seed}: iters "
        f"{info['iters']} vs {ref_it}, h relerr {e:.2e}")
    assert info["iters"] == ref_it and e <= 1e-5
    # and the backward at the GPU's solution
    g = I.series(seed, "g", ("normal", 0.0, 1.0), np.arange(B * D), T, np.float32)
    grads_vs_oracle(x, h.cpu().numpy(), g.reshape(B, D, T), B, D, T,
                    f"random deer bwd {B}x{D}x{T} seed={seed}")


@cases(15)
@given(B=st.integers(1, 3), D=st.integers(1, 200), T=layer_steps,
       io=st.sampled_from(["bf16", "f32"]), k_max=st.integers(1, 6), c0=st.booleans(),
       seed=seeds)
def test_sru_deer_random(B, D, T, io, k_max, c0, seed):
    assume(B * D * T <= MAX_ELEMS // 2)
    w = I.scaled(I.WORKLOADS["sru_deer"], B=B, D=D, T=T, seed=seed)
    c0v = np.random.default_rng(seed).normal(size=(B, D)).astype(np.float32) if c0 else None
    got, ref = sru_nl_run(w, io, c0v, k_max=k_max)
    assume(robust_count(ref[3], 1e-5))
    sru_nl_check(got, ref, io, f"random sru-deer {io} {B}x{D}x{T} k_max={k_max} seed={seed}")
