"""Pins for the oracle's SRU layer whose forget gate reads the previous cell
state (page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优", SRU
paragraph, the v_f (.) c_{t-1} term) and for its DEER solve (page
"cuda-parallel-rnn-training-logt-optimization", core principle and
engineering sections).

The sequential loop is pinned to the linear SRU oracle at v_f = 0 (bit for
bit) and to a 50-digit decimal evaluation; the Newton solve is pinned to the
sequential loop at convergence, to the exact-prefix property of Newton on a
causal recurrence, to the linear case (one step solves it), to quadratic
convergence, and, for one step from an arbitrary iterate, to the linearised
recurrence built from the sequential loop itself with a finite-difference
Jacobian (which pins both J and the right-hand side).
"""
import numpy as np
import pytest

from conftest import relerr
from decimal_ref import D, dsigmoid, dtanh


def case(seed, T=6, B=2, Dd=3, vs=0.25):
    rng = np.random.default_rng(seed)
    z = [rng.normal(size=(T, B, Dd)) for _ in range(3)]
    return dict(zf=z[0], zr=z[1], zx=z[2], bf=rng.normal(-1, 0.1, Dd), br=rng.normal(-1, 0.1, Dd),
                vf=rng.uniform(-vs, vs, Dd), c0=rng.normal(size=(B, Dd)))


def args(x, keys=("zf", "zr", "zx", "bf", "br", "vf")):
    return [x[k] for k in keys]


def test_linear_case_is_the_sru_layer(oracle_mod):
    x = case(1)
    h, c = oracle_mod.sru_nl_seq(*args(x)[:5], np.zeros(3), x["c0"])
    h_lin, c_last = oracle_mod.sru_fwd(*args(x)[:5], x["c0"])
    assert np.array_equal(h, h_lin)
    assert np.array_equal(c[-1], c_last)


def test_sequential_decimal(oracle_mod):
    x = case(2, vs=1.0)
    h, c = oracle_mod.sru_nl_seq(*args(x), x["c0"])
    T, B, Dd = x["zf"].shape
    for b in range(B):
        for d in range(Dd):
            s = D(x["c0"][b, d])
            for t in range(T):
                f = dsigmoid(D(x["zf"][t, b, d]) + D(x["bf"][d]) + D(x["vf"][d]) * s)
                r = dsigmoid(D(x["zr"][t, b, d]) + D(x["br"][d]))
                zx = D(x["zx"][t, b, d])
                s = f * s + (1 - f) * zx
                assert abs(float(s) - c[t, b, d]) < 1e-14 * (1 + abs(float(s)))
                ref = float(r * dtanh(s) + (1 - r) * zx)
                assert abs(ref - h[t, b, d]) < 1e-14 * (1 + abs(ref))


@pytest.mark.parametrize("vs", [0.25, 1.0])
def test_deer_converges_to_sequential(oracle_mod, vs):
    x = case(3, T=300, B=2, Dd=4, vs=vs)
    h_seq, c_seq = oracle_mod.sru_nl_seq(*args(x), x["c0"])
    h, c, iters, deltas = oracle_mod.sru_deer(*args(x), x["c0"], eps=1e-12, k_max=40)
    assert deltas[-1] < 1e-12 and iters < 40
    assert relerr(c, c_seq) < 1e-12 and relerr(h, h_seq) < 1e-12


def test_linear_case_one_newton_step(oracle_mod):
    """v_f = 0: the map is affine, so the first step is exact and the second
    changes nothing (delta_2 = 0)."""
    x = case(4, T=50)
    x["vf"] = np.zeros(3)
    h, c, iters, deltas = oracle_mod.sru_deer(*args(x), x["c0"], eps=1e-300, k_max=5)
    _, c_seq = oracle_mod.sru_nl_seq(*args(x), x["c0"])
    assert iters == 5 and np.all(deltas[1:] < 1e-13)
    assert relerr(c, c_seq) < 1e-14


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_exact_prefix(oracle_mod, k):
    """After k Newton steps from any start, steps 0..k-1 are exact (each step
    makes one more leading step exact on a causal recurrence)."""
    x = case(5, T=10, vs=1.0)
    rng = np.random.default_rng(50 + k)
    start = rng.normal(size=x["zf"].shape)
    _, c, iters, _ = oracle_mod.sru_deer(*args(x), x["c0"], c_init=start, eps=0.0, k_max=k)
    _, c_seq = oracle_mod.sru_nl_seq(*args(x), x["c0"])
    assert iters == k
    assert relerr(c[:k], c_seq[:k]) < 1e-13
    if k == 1:
        assert relerr(c[k:], c_seq[k:]) > 1e-6  # one step from a random start: the rest is off


def test_quadratic_convergence(oracle_mod):
    x = case(6, T=400, B=2, Dd=8, vs=1.0)
    _, _, _, d = oracle_mod.sru_deer(*args(x), x["c0"], eps=1e-13, k_max=30)
    # pairs above the rounding floor (50 d^2 well above 1e-16)
    tail = [(d[i], d[i + 1]) for i in range(len(d) - 1) if 1e-7 < d[i] < 1e-2]
    assert tail, d
    for a, b in tail:
        assert b < 50 * a * a, (a, b)


def test_one_step_is_the_linearised_recurrence(oracle_mod):
    """y' = J y'_{t-1} + F(y_{t-1}) - J y_{t-1}, with F evaluated by the
    sequential loop on one step started from y_{t-1} and J its central
    finite difference."""
    x = case(7, T=6, vs=1.0)
    rng = np.random.default_rng(70)
    y = rng.normal(size=x["zf"].shape)
    _, yn, _, _ = oracle_mod.sru_deer(*args(x), x["c0"], c_init=y, eps=0.0, k_max=1)

    def F(t, cprev):
        sl = [v[t:t + 1] for v in (x["zf"], x["zr"], x["zx"])]
        return oracle_mod.sru_nl_seq(*sl, x["bf"], x["br"], x["vf"], cprev)[1][0]
    step = 1e-6
    prev_new, prev_old = x["c0"], x["c0"]
    for t in range(y.shape[0]):
        J = (F(t, prev_old + step) - F(t, prev_old - step)) / (2 * step)
        want = J * prev_new + F(t, prev_old) - J * prev_old
        assert np.max(np.abs(yn[t] - want)) < 1e-8, t
        prev_new, prev_old = yn[t], y[t]


def test_stop_rule(oracle_mod):
    """Strict delta < eps and the k_max cap, as for the tanh RNN solve."""
    x = case(8, T=100, vs=1.0)
    _, _, it_all, d_all = oracle_mod.sru_deer(*args(x), x["c0"], eps=0.0, k_max=6)
    assert it_all == 6
    eps = float(d_all[2])  # equal to delta_3: not below it, so the solve goes on
    _, _, it, d = oracle_mod.sru_deer(*args(x), x["c0"], eps=eps, k_max=6)
    assert it == 4 and np.array_equal(d, d_all[:4])
