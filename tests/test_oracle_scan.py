"""Pins for the oracle's forward scan and its reverse-time adjoint.

Each check ties the oracle to something other than itself: a closed form, a
library prefix sum, an exact rational evaluation of the unrolled product-sum
expansion (a different formula from the recurrence), an adjoint identity, or
central finite differences of the forward map.  The mistakes they are chosen
to catch: a dropped or doubled term, an off-by-one in time (h_{t-1} vs h_t,
a_t vs a_{t+1}), a wrong h0 fold, a transposed operand in the combine, and a
wrong dh0.
"""
from fractions import Fraction

import numpy as np
import pytest

from conftest import relerr


def dyadic(rng, shape, lo, hi, bits=10):
    """Random values that are exact binary fractions (exact in fp64 and Fraction)."""
    return np.round(rng.uniform(lo, hi, shape) * (1 << bits)) / (1 << bits)


# ---------------------------------------------------------------- forward

def test_constant_a_geometric_closed_form(oracle_mod):
    T, c, beta, h0 = 300, 0.97, 0.25, 1.5
    a = np.full((1, T), c)
    b = np.full((1, T), beta)
    h = oracle_mod.scan_fwd(a, b, np.array([h0]))
    t = np.arange(1, T + 1, dtype=np.float64)
    closed = c ** t * h0 + beta * (1 - c ** t) / (1 - c)
    assert relerr(h[0], closed) < 1e-13


def test_constant_a_arbitrary_b_closed_form(oracle_mod):
    rng = np.random.default_rng(7)
    T, c = 64, 0.9
    b = rng.normal(size=(1, T))
    h = oracle_mod.scan_fwd(np.full((1, T), c), b, np.array([0.0]))
    # h_t = sum_k c^(t-k) b_k, evaluated as a Toeplitz matrix-vector product
    k = np.arange(T)
    M = np.tril(c ** (k[:, None] - k[None, :]).astype(np.float64))
    assert relerr(h[0], M @ b[0]) < 1e-13


def test_a_one_is_prefix_sum(oracle_mod):
    rng = np.random.default_rng(1)
    b = rng.normal(size=(3, 500))
    h0 = rng.normal(size=3)
    h = oracle_mod.scan_fwd(np.ones_like(b), b, h0)
    assert relerr(h, h0[:, None] + np.cumsum(b, axis=1)) < 1e-13


def test_a_zero_gives_b(oracle_mod):
    rng = np.random.default_rng(2)
    b = rng.normal(size=(4, 33))
    h = oracle_mod.scan_fwd(np.zeros_like(b), b, rng.normal(size=4))
    assert np.array_equal(h, b)


def unrolled_fraction(a, b, h0):
    """h_t = (prod_{k<=t} a_k) h0 + sum_{k<=t} (prod_{k<j<=t} a_j) b_k, exactly."""
    T = len(a)
    A = [Fraction(float(x)) for x in a]
    Bv = [Fraction(float(x)) for x in b]
    out = []
    for t in range(T):
        p = Fraction(1)
        for j in range(t + 1):
            p *= A[j]
        acc = p * Fraction(float(h0))
        for k in range(t + 1):
            p = Fraction(1)
            for j in range(k + 1, t + 1):
                p *= A[j]
            acc += p * Bv[k]
        out.append(acc)
    return out


@pytest.mark.parametrize("T", [1, 2, 5, 16])
def test_forward_exact_bruteforce(oracle_mod, T):
    rng = np.random.default_rng(100 + T)
    C = 3
    a = dyadic(rng, (C, T), -1.2, 1.2)
    b = dyadic(rng, (C, T), -2, 2)
    h0 = dyadic(rng, (C,), -1, 1)
    h = oracle_mod.scan_fwd(a, b, h0)
    for c in range(C):
        exact = unrolled_fraction(a[c], b[c], h0[c])
        ref = np.array([float(x) for x in exact])
        assert relerr(h[c], ref) < 1e-14


def test_split_and_continue(oracle_mod):
    """Scanning [0,T) equals scanning [0,k) then [k,T) from h_k: pins the h0 fold."""
    rng = np.random.default_rng(3)
    a = rng.uniform(0.5, 1.0, (2, 200))
    b = rng.normal(size=(2, 200))
    h0 = rng.normal(size=2)
    full = oracle_mod.scan_fwd(a, b, h0)
    k = 77
    first = oracle_mod.scan_fwd(a[:, :k], b[:, :k], h0)
    second = oracle_mod.scan_fwd(a[:, k:], b[:, k:], first[:, -1])
    assert np.array_equal(np.concatenate([first, second], axis=1), full)


def test_null_h0_is_zero(oracle_mod):
    rng = np.random.default_rng(4)
    a = rng.uniform(size=(2, 9))
    b = rng.normal(size=(2, 9))
    assert np.array_equal(oracle_mod.scan_fwd(a, b, None), oracle_mod.scan_fwd(a, b, np.zeros(2)))


def test_leading_dims_are_channels(oracle_mod):
    rng = np.random.default_rng(5)
    a = rng.uniform(size=(2, 3, 11))
    b = rng.normal(size=(2, 3, 11))
    h0 = rng.normal(size=(2, 3))
    h = oracle_mod.scan_fwd(a, b, h0)
    for i in range(2):
        for j in range(3):
            assert np.array_equal(h[i, j], oracle_mod.scan_fwd(a[i, j][None], b[i, j][None],
                                                              h0[i, j:j + 1])[0])


# ---------------------------------------------------------------- backward

def test_adjoint_identity(oracle_mod):
    """h is linear in (b, h0) for fixed a, so <g, h> = <lam, b> + dh0*h0 per channel."""
    rng = np.random.default_rng(6)
    C, T = 5, 400
    a = rng.uniform(0.8, 0.999, (C, T))
    b = rng.normal(size=(C, T))
    g = rng.normal(size=(C, T))
    h0 = rng.normal(size=C)
    h = oracle_mod.scan_fwd(a, b, h0)
    da, db, dh0 = oracle_mod.scan_bwd(a, h, h0, g)
    lhs = np.sum(g * h, axis=1)
    rhs = np.sum(db * b, axis=1) + dh0 * h0
    assert np.max(np.abs(lhs - rhs) / (1 + np.abs(lhs))) < 1e-12


def test_finite_differences(oracle_mod):
    """Central differences of L = <g, h(a, b, h0)> in fp64."""
    rng = np.random.default_rng(8)
    T = 12
    a = rng.uniform(0.3, 1.1, (1, T))
    b = rng.normal(size=(1, T))
    g = rng.normal(size=(1, T))
    h0 = rng.normal(size=1)

    def L(a_, b_, h0_):
        return float(np.sum(g * oracle_mod.scan_fwd(a_, b_, h0_)))

    h = oracle_mod.scan_fwd(a, b, h0)
    da, db, dh0 = oracle_mod.scan_bwd(a, h, h0, g)
    eps = 1e-6
    for t in range(T):
        e = np.zeros_like(a)
        e[0, t] = eps
        fd_a = (L(a + e, b, h0) - L(a - e, b, h0)) / (2 * eps)
        fd_b = (L(a, b + e, h0) - L(a, b - e, h0)) / (2 * eps)
        assert abs(fd_a - da[0, t]) < 1e-7 * (1 + abs(da[0, t]))
        assert abs(fd_b - db[0, t]) < 1e-7 * (1 + abs(db[0, t]))
    fd_h0 = (L(a, b, h0 + eps) - L(a, b, h0 - eps)) / (2 * eps)
    assert abs(fd_h0 - dh0[0]) < 1e-7 * (1 + abs(dh0[0]))


@pytest.mark.parametrize("T", [1, 3, 9])
def test_backward_exact_bruteforce(oracle_mod, T):
    """Exact gradients from the expansion dh_s/da_t = h_{t-1} prod_{t<j<=s} a_j."""
    rng = np.random.default_rng(200 + T)
    a = dyadic(rng, (1, T), -1.2, 1.2)
    b = dyadic(rng, (1, T), -2, 2)
    g = dyadic(rng, (1, T), -2, 2)
    h0 = dyadic(rng, (1,), -1, 1)
    hx = unrolled_fraction(a[0], b[0], h0[0])
    A = [Fraction(float(x)) for x in a[0]]
    G = [Fraction(float(x)) for x in g[0]]
    hprev = [Fraction(float(h0[0]))] + hx[:-1]
    db_ref, da_ref = [], []
    for t in range(T):
        lam = Fraction(0)
        for s in range(t, T):
            p = Fraction(1)
            for j in range(t + 1, s + 1):
                p *= A[j]
            lam += G[s] * p
        db_ref.append(lam)
        da_ref.append(lam * hprev[t])
    dh0_ref = A[0] * db_ref[0]
    h = np.array([[float(x) for x in hx]])
    da, db, dh0 = oracle_mod.scan_bwd(a, h, h0, g)
    assert relerr(db[0], [float(x) for x in db_ref]) < 1e-14
    assert relerr(da[0], [float(x) for x in da_ref]) < 1e-14
    assert abs(dh0[0] - float(dh0_ref)) < 1e-14 * (1 + abs(float(dh0_ref)))


def test_backward_a_one_reverse_cumsum(oracle_mod):
    rng = np.random.default_rng(9)
    g = rng.normal(size=(2, 300))
    b = rng.normal(size=(2, 300))
    h0 = rng.normal(size=2)
    a = np.ones_like(g)
    h = oracle_mod.scan_fwd(a, b, h0)
    da, db, dh0 = oracle_mod.scan_bwd(a, h, h0, g)
    lam = np.cumsum(g[:, ::-1], axis=1)[:, ::-1]
    assert relerr(db, lam) < 1e-13
    hprev = np.concatenate([h0[:, None], h[:, :-1]], axis=1)
    assert relerr(da, lam * hprev) < 1e-13
    assert relerr(dh0, lam[:, 0]) < 1e-13


def test_backward_a_zero(oracle_mod):
    rng = np.random.default_rng(10)
    g = rng.normal(size=(2, 50))
    h = rng.normal(size=(2, 50))
    h0 = rng.normal(size=2)
    da, db, dh0 = oracle_mod.scan_bwd(np.zeros_like(g), h, h0, g)
    assert np.array_equal(db, g)
    hprev = np.concatenate([h0[:, None], h[:, :-1]], axis=1)
    assert np.array_equal(da, g * hprev)
    assert np.array_equal(dh0, np.zeros(2))


def test_planted_mistake_is_caught(oracle_mod):
    """A copy of the recurrence with a deliberate off-by-one in a (a_{t+1} used at step t)
    fails the exact brute force; guards the brute force itself against being vacuous."""
    rng = np.random.default_rng(11)
    T = 6
    a = dyadic(rng, (T,), 0.3, 1.1)
    b = dyadic(rng, (T,), -2, 2)
    exact = np.array([float(x) for x in unrolled_fraction(a, b, 0.5)])
    wrong = []
    s = 0.5
    for t in range(T):
        s = (a[t + 1] if t + 1 < T else a[t]) * s + b[t]
        wrong.append(s)
    assert relerr(np.array(wrong), exact) > 1e-6
    assert relerr(oracle_mod.scan_fwd(a[None], b[None], np.array([0.5]))[0], exact) < 1e-14
