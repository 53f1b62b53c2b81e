"""Pins for the oracle's SRU layer (page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优",
body, SRU paragraph; gates without the v_f*c_{t-1} term).

Limits of the gates fix which gate does what (f vs 1-f, r vs 1-r, bias per
feature d and not per batch entry), the f = r = 1/2 case is exact binary
arithmetic for the cell state, and tanh/sigmoid are checked against decimal's
own exp(), which does not go through the C math library the oracle uses.
"""
import numpy as np

from conftest import relerr
from decimal_ref import D, dsigmoid, dtanh

BIG = 800.0  # sigma(+-800) is exactly 1 / 0 in fp64


def zeros(T, B, Dd):
    return np.zeros((T, B, Dd))


def test_forget_gate_closed_keeps_state(oracle_mod):
    """b_f = +800: f = 1, c_t = c_0 for all t; with b_r = -800, r = 0 so h = z_x."""
    rng = np.random.default_rng(1)
    T, B, Dd = 7, 2, 3
    zx = rng.normal(size=(T, B, Dd))
    zf = rng.normal(size=(T, B, Dd))
    zr = rng.normal(size=(T, B, Dd))
    c0 = rng.normal(size=(B, Dd))
    h, c_last = oracle_mod.sru_fwd(zf, zr, zx, np.full(Dd, BIG), np.full(Dd, -BIG), c0)
    assert np.array_equal(h, zx)
    assert np.array_equal(c_last, c0)


def test_forget_gate_open_copies_candidate(oracle_mod):
    """b_f = -800: f = 0, c_t = z_x,t; with b_r = +800, r = 1 so h = tanh(z_x)."""
    rng = np.random.default_rng(2)
    T, B, Dd = 5, 2, 2
    zx = rng.normal(size=(T, B, Dd))
    h, c_last = oracle_mod.sru_fwd(rng.normal(size=zx.shape), rng.normal(size=zx.shape), zx,
                                   np.full(Dd, -BIG), np.full(Dd, BIG))
    ref = np.vectorize(lambda v: float(dtanh(D(v))))(zx)
    assert relerr(h, ref) < 1e-15
    assert np.array_equal(c_last, zx[-1])


def test_bias_is_per_feature(oracle_mod):
    """Feature 0 has f=1 (state kept at c0), feature 1 has f=0 (state = z_x):
    a bias indexed by batch entry instead of feature would mix them."""
    rng = np.random.default_rng(3)
    T, B, Dd = 4, 3, 2
    zx = rng.normal(size=(T, B, Dd))
    c0 = rng.normal(size=(B, Dd))
    h, c_last = oracle_mod.sru_fwd(zeros(T, B, Dd), zeros(T, B, Dd), zx,
                                   np.array([BIG, -BIG]), np.array([-BIG, -BIG]), c0)
    assert np.array_equal(c_last[:, 0], c0[:, 0])
    assert np.array_equal(c_last[:, 1], zx[-1, :, 1])
    assert np.array_equal(h, zx)


def test_half_gates_exact(oracle_mod):
    """z_f = -b_f and z_r = -b_r give f = r = 1/2 exactly: c_t = (c_{t-1} + z_x,t)/2 in
    exact binary arithmetic, h_t = tanh(c_t)/2 + z_x,t/2."""
    T, B, Dd = 4, 1, 1
    zx = np.array([2.0, 4.0, 8.0, -6.0]).reshape(T, B, Dd)
    bf = np.array([-1.0])
    br = np.array([0.75])
    zf = np.full((T, B, Dd), 1.0)
    zr = np.full((T, B, Dd), -0.75)
    h, c_last = oracle_mod.sru_fwd(zf, zr, zx, bf, br)
    c_exact = [1.0, 2.5, 5.25, -0.375]  # (0+2)/2, (1+4)/2, (2.5+8)/2, (5.25-6)/2
    assert c_last[0, 0] == c_exact[-1]
    ref = [float(dtanh(D(c)) / 2 + D(z) / 2) for c, z in zip(c_exact, zx.ravel())]
    assert relerr(h.ravel(), ref) < 1e-15


def test_decimal_bruteforce_small(oracle_mod):
    """Whole layer at T=6, B=2, D=3 against a 50-digit decimal evaluation of the
    gates (independent exp/tanh implementation)."""
    rng = np.random.default_rng(4)
    T, B, Dd = 6, 2, 3
    zf, zr, zx = (rng.normal(size=(T, B, Dd)) for _ in range(3))
    bf = rng.normal(-1, 0.1, Dd)
    br = rng.normal(-1, 0.1, Dd)
    c0 = rng.normal(size=(B, Dd))
    h, c_last = oracle_mod.sru_fwd(zf, zr, zx, bf, br, c0)
    ref = np.empty_like(h)
    cl = np.empty_like(c_last)
    for b in range(B):
        for d in range(Dd):
            c = D(c0[b, d])
            for t in range(T):
                f = dsigmoid(D(zf[t, b, d]) + D(bf[d]))
                r = dsigmoid(D(zr[t, b, d]) + D(br[d]))
                x = D(zx[t, b, d])
                c = f * c + (1 - f) * x
                ref[t, b, d] = float(r * dtanh(c) + (1 - r) * x)
            cl[b, d] = float(c)
    assert relerr(h, ref) < 1e-14
    assert relerr(c_last, cl) < 1e-14
