"""Pins for the oracle's LSTM cell-state layer with input-only gates (page
"RNN CUDA内核优化：实现序列长度无关的恒定推理延迟", body: the LSTM cell state
C_t = f_t*C_{t-1} + i_t*C~_t as a linear recurrence, and the deployment list's
model-change step) and its backward (chain rule; the cell-state gradient is a
reverse-time linear recurrence, page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优",
parallel-scan paragraph).

Forward: saturated gates fix which pre-activation drives which gate (f keeps
the state, i admits the candidate, o scales the output), the f = 1 limit turns
the cell state into a running sum, and a 50-digit decimal evaluation checks
the whole layer with an exp() that does not come from the C math library.
Backward: central finite differences of L = sum(gh*h) + sum(gcl*c_T) through
the (pinned) forward for every input entry, plus closed forms in the
saturated limits.
"""
import numpy as np
import pytest

from conftest import relerr
from decimal_ref import D, dsigmoid, dtanh

BIG = 800.0  # sigma(+-800) is exactly 1 / 0 in fp64


def rand(rng, T, B, Dd, n):
    return [rng.normal(size=(T, B, Dd)) for _ in range(n)]


def test_forget_shut_input_open_is_running_sum(oracle_mod):
    """f = 1, i = 1: c_t = c0 + sum_{s<=t} tanh(z_c,s); o = 1: h = tanh(c)."""
    rng = np.random.default_rng(11)
    T, B, Dd = 9, 2, 3
    zc = rng.normal(size=(T, B, Dd))
    c0 = rng.normal(size=(B, Dd))
    full = np.full((T, B, Dd), BIG)
    h, c_last = oracle_mod.lstm_fwd(full, full, zc, full, c0)
    c = c0[None] + np.cumsum(np.tanh(zc), axis=0)
    assert relerr(h, np.tanh(c)) < 1e-14
    assert relerr(c_last, c[-1]) < 1e-14


def test_input_gate_shut_keeps_decayed_state(oracle_mod):
    """i = 0: c_t = c0 * prod f (nothing from z_c); o = 0 gives h = 0."""
    rng = np.random.default_rng(12)
    T, B, Dd = 6, 2, 2
    zf, zc = rand(rng, T, B, Dd, 2)
    c0 = rng.normal(size=(B, Dd))
    h, c_last = oracle_mod.lstm_fwd(zf, np.full_like(zf, -BIG), zc, np.full_like(zf, -BIG), c0)
    f = 1.0 / (1.0 + np.exp(-zf))
    assert np.array_equal(h, np.zeros_like(h))
    assert relerr(c_last, c0 * np.prod(f, axis=0)) < 1e-14


def test_forget_gate_open_forgets(oracle_mod):
    """f = 0: each step stands alone, c_t = i_t tanh(z_c,t); c0 has no effect."""
    rng = np.random.default_rng(13)
    T, B, Dd = 5, 3, 2
    zi, zc, zo = rand(rng, T, B, Dd, 3)
    h1, c1 = oracle_mod.lstm_fwd(np.full_like(zi, -BIG), zi, zc, zo, rng.normal(size=(B, Dd)))
    h2, c2 = oracle_mod.lstm_fwd(np.full_like(zi, -BIG), zi, zc, zo)
    assert np.array_equal(h1, h2) and np.array_equal(c1, c2)
    i = 1.0 / (1.0 + np.exp(-zi))
    o = 1.0 / (1.0 + np.exp(-zo))
    assert relerr(h1, o * np.tanh(i * np.tanh(zc))) < 1e-15


def test_half_gates_exact(oracle_mod):
    """z_f = z_i = 0 gives f = i = 1/2 exactly, and z_c with tanh(z_c) known to
    50 digits: c_t = (c_{t-1} + tanh z_c,t)/2 evaluated in decimal."""
    zc = np.array([0.5, -1.25, 2.0, 0.0]).reshape(4, 1, 1)
    zero = np.zeros_like(zc)
    h, c_last = oracle_mod.lstm_fwd(zero, zero, zc, np.full_like(zc, BIG), np.array([[3.0]]))
    c = D(3.0)
    ref = []
    for z in zc.ravel():
        c = (c + dtanh(D(z))) / 2
        ref.append(float(dtanh(c)))
    assert relerr(h.ravel(), ref) < 1e-15
    assert relerr(c_last.ravel(), [float(c)]) < 1e-15


def test_decimal_bruteforce_small(oracle_mod):
    """Whole layer at T=6, B=2, D=3 against a 50-digit decimal evaluation."""
    rng = np.random.default_rng(14)
    T, B, Dd = 6, 2, 3
    zf, zi, zc, zo = rand(rng, T, B, Dd, 4)
    c0 = rng.normal(size=(B, Dd))
    h, c_last = oracle_mod.lstm_fwd(zf, zi, zc, zo, c0)
    ref = np.empty_like(h)
    cl = np.empty_like(c_last)
    for b in range(B):
        for d in range(Dd):
            c = D(c0[b, d])
            for t in range(T):
                f = dsigmoid(D(zf[t, b, d]))
                i = dsigmoid(D(zi[t, b, d]))
                g = dtanh(D(zc[t, b, d]))
                o = dsigmoid(D(zo[t, b, d]))
                c = f * c + i * g
                ref[t, b, d] = float(o * dtanh(c))
            cl[b, d] = float(c)
    assert relerr(h, ref) < 1e-14
    assert relerr(c_last, cl) < 1e-14


# ---- backward ---------------------------------------------------------------

NAMES = ("zf", "zi", "zc", "zo")


def loss(o, x, **over):
    v = {**x, **over}
    h, c_last = o.lstm_fwd(v["zf"], v["zi"], v["zc"], v["zo"], v["c0"])
    return float(np.sum(v["gh"] * h) + np.sum(v["gcl"] * c_last))


def case(seed, T=4, B=2, Dd=3):
    rng = np.random.default_rng(seed)
    x = dict(zip(NAMES, rand(rng, T, B, Dd, 4)))
    return dict(x, c0=rng.normal(size=(B, Dd)), gh=rng.normal(size=(T, B, Dd)),
                gcl=rng.normal(size=(B, Dd)))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_bwd_finite_differences(oracle_mod, seed):
    x = case(seed)
    g = oracle_mod.lstm_bwd(x["zf"], x["zi"], x["zc"], x["zo"], x["gh"], c0=x["c0"], gcl=x["gcl"])
    step = 1e-6
    for name in NAMES + ("c0",):
        base = x[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += step
            minus[idx] -= step
            fd[idx] = (loss(oracle_mod, x, **{name: plus}) -
                       loss(oracle_mod, x, **{name: minus})) / (2 * step)
        err = np.max(np.abs(g["d" + name] - fd)) / (1 + np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_bwd_forget_shut_is_reverse_running_sum(oracle_mod):
    """f = 1: gc_t = gcl + sum_{s>=t} gh_s o_s (1 - tanh^2 c_s), dz_f = 0,
    dc0 = gc_1, dz_c = gc_t i_t (1 - tanh^2 z_c,t)."""
    x = case(21, T=7)
    zf = np.full_like(x["zf"], BIG)
    g = oracle_mod.lstm_bwd(zf, x["zi"], x["zc"], x["zo"], x["gh"], c0=x["c0"], gcl=x["gcl"])
    i = 1.0 / (1.0 + np.exp(-x["zi"]))
    o = 1.0 / (1.0 + np.exp(-x["zo"]))
    c = x["c0"][None] + np.cumsum(i * np.tanh(x["zc"]), axis=0)
    e = x["gh"] * o * (1 - np.tanh(c) ** 2)
    gc = x["gcl"][None] + np.cumsum(e[::-1], axis=0)[::-1]
    assert np.array_equal(g["dzf"], np.zeros_like(g["dzf"]))
    assert relerr(g["dc0"], gc[0]) < 1e-14
    assert relerr(g["dzc"], gc * i * (1 - np.tanh(x["zc"]) ** 2)) < 1e-14
    assert relerr(g["dzo"], x["gh"] * np.tanh(c) * o * (1 - o)) < 1e-14


def test_bwd_output_gate_shut(oracle_mod):
    """o = 0: h does not depend on anything, so only dL/dc_T flows:
    gc_t = gcl * prod_{s>t} f_s, dz_o = 0, dc0 = gcl * prod f."""
    x = case(22, T=5)
    zo = np.full_like(x["zo"], -BIG)
    g = oracle_mod.lstm_bwd(x["zf"], x["zi"], x["zc"], zo, x["gh"], c0=x["c0"], gcl=x["gcl"])
    f = 1.0 / (1.0 + np.exp(-x["zf"]))
    assert np.array_equal(g["dzo"], np.zeros_like(g["dzo"]))
    assert relerr(g["dc0"], x["gcl"] * np.prod(f, axis=0)) < 1e-14
    # the last step's cell-state gradient is gcl itself
    i = 1.0 / (1.0 + np.exp(-x["zi"][-1]))
    assert relerr(g["dzc"][-1], x["gcl"] * i * (1 - np.tanh(x["zc"][-1]) ** 2)) < 1e-14
