"""Pins for the oracle's sequential nonlinear RNN and its DEER Newton solve
(DEER page, sections "核心原理" and "工程实现").

* the sequential loop h_t = tanh(w h_{t-1} + u_t) against decimal's exp();
* w = 0: the Jacobian vanishes, one iteration gives tanh(u) exactly and the
  second iteration changes nothing;
* exact-prefix invariant: h_0 is fixed, so iteration k reproduces the
  sequential solution exactly on steps 1..k;
* a converged run equals the sequential loop; late iterations converge
  quadratically;
* one Newton step solves the linearised residual equation, with the
  Jacobian taken by finite differences of tanh (pins J and the right-hand side);
* the stop rule: strict "<" against eps, K_max cap, the pages' constants.
"""
import os

import numpy as np
import pytest

from conftest import relerr
from decimal_ref import D, dtanh

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def make(seed, B=2, Dd=3, T=40, wmax=0.9):
    rng = np.random.default_rng(seed)
    return rng.uniform(-wmax, wmax, Dd), rng.normal(size=(B, Dd, T)), rng.normal(size=(B, Dd))


def test_sequential_loop_decimal(oracle_mod):
    w, u, h0 = make(1, T=8)
    h = oracle_mod.rnn_seq(w, u, h0)
    B, Dd, T = u.shape
    ref = np.empty_like(h)
    for b in range(B):
        for d in range(Dd):
            s = D(h0[b, d])
            for t in range(T):
                s = dtanh(D(w[d]) * s + D(u[b, d, t]))
                ref[b, d, t] = float(s)
    assert relerr(h, ref) < 1e-14


def test_w_zero_one_step(oracle_mod):
    _, u, h0 = make(2)
    w = np.zeros(u.shape[1])
    h, iters, deltas = oracle_mod.deer(w, u, h0, eps=1e-5, k_max=5)
    ref = np.vectorize(lambda v: float(dtanh(D(v))))(u)
    assert relerr(h, ref) < 1e-15
    assert iters == 2 and deltas[1] == 0.0 and deltas[0] > 1e-5


def test_exact_prefix_invariant(oracle_mod):
    w, u, h0 = make(3, T=30)
    seq = oracle_mod.rnn_seq(w, u, h0)
    for k in range(1, 6):
        h, iters, _ = oracle_mod.deer(w, u, h0, eps=0.0, k_max=k)
        assert iters == k
        assert np.max(np.abs(h[..., :k] - seq[..., :k])) < 1e-14
        # and step k+1 is in general not yet exact
        assert np.max(np.abs(h[..., k:k + 1] - seq[..., k:k + 1])) > 0


def test_converges_to_sequential(oracle_mod):
    w, u, h0 = make(4, T=200)
    seq = oracle_mod.rnn_seq(w, u, h0)
    h, iters, deltas = oracle_mod.deer(w, u, h0, eps=1e-13, k_max=60)
    assert deltas[-1] < 1e-13 and iters < 60
    assert relerr(h, seq) < 1e-12


def test_quadratic_convergence(oracle_mod):
    w, u, h0 = make(5, B=4, Dd=8, T=300)
    _, iters, deltas = oracle_mod.deer(w, u, h0, eps=1e-14, k_max=40)
    late = [(deltas[i], deltas[i + 1]) for i in range(iters - 1) if 1e-12 < deltas[i + 1] and deltas[i] < 1e-1]
    assert late, deltas
    for d0, d1 in late:
        assert d1 <= 10.0 * d0 * d0, (d0, d1, deltas)


def test_newton_step_solves_linearised_residual(oracle_mod):
    """From any iterate y, one iteration y' satisfies
    (y'_t - y_t) - J_t (y'_{t-1} - y_{t-1}) = -(y_t - tanh(w y_{t-1} + u_t)),
    with J_t the derivative of tanh(w x + u_t) at x = y_{t-1} (finite differences)."""
    w, u, h0 = make(6, T=25)
    rng = np.random.default_rng(60)
    y = rng.normal(scale=0.5, size=u.shape)
    y1, iters, _ = oracle_mod.deer(w, u, h0, h_init=y, eps=0.0, k_max=1)
    assert iters == 1
    yprev = np.concatenate([h0[..., None], y[..., :-1]], axis=-1)
    y1prev = np.concatenate([h0[..., None], y1[..., :-1]], axis=-1)
    wf = w[None, :, None]
    eps = 1e-6
    J = (np.tanh(wf * (yprev + eps) + u) - np.tanh(wf * (yprev - eps) + u)) / (2 * eps)
    F = y - np.tanh(wf * yprev + u)
    lhs = (y1 - y) - J * (y1prev - yprev)
    assert np.max(np.abs(lhs + F)) < 1e-8


def test_stop_rule_strict_and_capped(oracle_mod):
    w, u, h0 = make(7)
    _, iters_all, deltas = oracle_mod.deer(w, u, h0, eps=0.0, k_max=4)
    assert iters_all == 4 and len(deltas) == 4
    # eps equal to delta_2 does not stop at 2 (strict <); slightly above it does
    _, it_eq, _ = oracle_mod.deer(w, u, h0, eps=deltas[1], k_max=4)
    _, it_gt, _ = oracle_mod.deer(w, u, h0, eps=np.nextafter(deltas[1], np.inf), k_max=4)
    assert it_gt == 2 and it_eq > 2
    _, it_one, _ = oracle_mod.deer(w, u, h0, eps=1e9, k_max=4)
    assert it_one == 1


def test_nan_does_not_converge(oracle_mod):
    w, u, h0 = make(8)
    u = u.copy()
    u[0, 0, 5] = np.nan
    _, iters, deltas = oracle_mod.deer(w, u, h0, eps=1e-5, k_max=3)
    assert iters == 3 and all(np.isnan(deltas))


def test_pages_stop_constants():
    """The DEER page's engineering section gives eps = 1e-5 and K_max = 5 as the
    example stop rule; the fixture records them with their citation."""
    vals = {}
    with open(os.path.join(GOLDEN, "deer_stop_rule.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = float(v)
    assert vals == {"eps": 1e-5, "k_max": 5.0}
    from linear_recurrence_scan_diagonal_amd import DEER_DEFAULT_EPS, DEER_DEFAULT_KMAX
    assert DEER_DEFAULT_EPS == vals["eps"] and DEER_DEFAULT_KMAX == int(vals["k_max"])
