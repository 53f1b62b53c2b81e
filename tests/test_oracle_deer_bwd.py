"""Pins for the oracle's adjoint of the nonlinear RNN h_t = tanh(w h_{t-1} + u_t)
at its solution (DEER page "cuda-parallel-rnn-training-logt-optimization",
core principle: the solve's result is the sequential solution; the backward
pass as a reverse-time scan, page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优",
parallel-scan paragraph).

Central finite differences of L = sum(g * h(u, w, h0)), with h from the plain
sequential loop (pinned separately against decimal arithmetic), check du, dw
and dh0 for every entry; closed forms cover w = 0 (no coupling in time) and
the linear regime of small inputs.
"""
import numpy as np
import pytest


def case(seed, B=2, D=3, T=6):
    rng = np.random.default_rng(seed)
    return (rng.uniform(-0.9, 0.9, size=D), rng.normal(size=(B, D, T)),
            rng.normal(size=(B, D)), rng.normal(size=(B, D, T)))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_finite_differences(oracle_mod, seed):
    w, u, h0, g = case(seed)
    h = oracle_mod.rnn_seq(w, u, h0)
    du, dw, dh0 = oracle_mod.deer_bwd(w, h, g, h0)

    def L(w_, u_, h0_):
        return float(np.sum(g * oracle_mod.rnn_seq(w_, u_, h0_)))
    step = 1e-6
    for name, base, grad in (("u", u, du), ("w", w, dw), ("h0", h0, dh0)):
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += step
            m[idx] -= step
            args_p = {"w_": w, "u_": u, "h0_": h0}
            args_m = dict(args_p)
            key = {"u": "u_", "w": "w_", "h0": "h0_"}[name]
            args_p[key], args_m[key] = p, m
            fd[idx] = (L(**args_p) - L(**args_m)) / (2 * step)
        err = np.max(np.abs(grad - fd)) / (1 + np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_no_coupling_when_w_is_zero(oracle_mod):
    """w = 0: h_t = tanh(u_t), so dL/du_t = g_t (1 - tanh^2 u_t), dL/dh0 = 0,
    and dL/dw = sum_t g_t (1 - h_t^2) h_{t-1}."""
    _, u, h0, g = case(5, T=7)
    w = np.zeros(3)
    h = oracle_mod.rnn_seq(w, u, h0)
    du, dw, dh0 = oracle_mod.deer_bwd(w, h, g, h0)
    s = 1 - np.tanh(u) ** 2
    assert np.allclose(du, g * s, rtol=1e-14, atol=1e-15)
    assert np.array_equal(dh0, np.zeros_like(dh0))
    hprev = np.concatenate([h0[..., None], h[..., :-1]], axis=-1)
    assert np.allclose(dw, np.sum(g * s * hprev, axis=(0, 2)), rtol=1e-13, atol=1e-15)


def test_small_signal_is_the_linear_adjoint(oracle_mod):
    """With h = 0 everywhere (s = 1) the adjoint is the linear reverse scan with
    constant coefficient w: lam_t = sum_{k>=t} w^(k-t) g_k."""
    B, D, T = 1, 2, 9
    w = np.array([0.5, -0.25])
    h = np.zeros((B, D, T))
    g = np.random.default_rng(6).normal(size=(B, D, T))
    du, _, dh0 = oracle_mod.deer_bwd(w, h, g)
    for d in range(D):
        lam = [sum(w[d] ** (k - t) * g[0, d, k] for k in range(t, T)) for t in range(T)]
        assert np.allclose(du[0, d], lam, rtol=1e-14, atol=1e-15)
        assert np.isclose(dh0[0, d], w[d] * lam[0], rtol=1e-14)
