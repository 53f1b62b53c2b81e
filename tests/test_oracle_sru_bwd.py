"""Pins for the oracle's SRU backward (page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优",
body, SRU paragraph: the backward pass is also a scan; the formulas are the
chain rule of the forward layer).

The gradients are checked against central finite differences of the loss
L = sum(gh * h) + sum(gcl * c_T) evaluated with the forward oracle (itself
pinned against decimal arithmetic), which catches any dropped term, sign or
time index; and against closed forms when the forget gate is saturated shut
(c_t = c_0) or open (c_t = z_x,t).
"""
import numpy as np
import pytest

BIG = 800.0  # sigma(+-800) is exactly 1 / 0 in fp64


def loss(o, zf, zr, zx, bf, br, c0, gh, gcl):
    h, c_last = o.sru_fwd(zf, zr, zx, bf, br, c0)
    return float(np.sum(gh * h) + np.sum(gcl * c_last))


def case(seed, T=4, B=2, Dd=3):
    rng = np.random.default_rng(seed)
    z = {k: rng.normal(size=(T, B, Dd)) for k in ("zf", "zr", "zx")}
    return dict(z, bf=rng.normal(-1, 0.3, size=Dd), br=rng.normal(-1, 0.3, size=Dd),
                c0=rng.normal(size=(B, Dd)), gh=rng.normal(size=(T, B, Dd)),
                gcl=rng.normal(size=(B, Dd)))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_finite_differences(oracle_mod, seed):
    x = case(seed)
    g = oracle_mod.sru_bwd(x["zf"], x["zr"], x["zx"], x["bf"], x["br"], x["gh"], c0=x["c0"],
                           gcl=x["gcl"])
    step = 1e-6
    for name, grad in (("zf", "dzf"), ("zr", "dzr"), ("zx", "dzx"), ("bf", "dbf"),
                       ("br", "dbr"), ("c0", "dc0")):
        base = x[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += step
            minus[idx] -= step
            lp = loss(oracle_mod, **{**{k: x[k] for k in ("zf", "zr", "zx", "bf", "br", "c0",
                                                          "gh", "gcl")}, name: plus})
            lm = loss(oracle_mod, **{**{k: x[k] for k in ("zf", "zr", "zx", "bf", "br", "c0",
                                                          "gh", "gcl")}, name: minus})
            fd[idx] = (lp - lm) / (2 * step)
        err = np.max(np.abs(g[grad] - fd)) / (1 + np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_forget_gate_shut(oracle_mod):
    """b_f = +800: f = 1, so c_t = c_0 for every t, nothing flows through z_f or
    (1 - f) z_x, and dL/dc0 collects every step: gcl + sum_t gh_t r_t (1 - tanh^2 c0)."""
    x = case(7, T=6)
    bf = np.full(3, BIG)
    g = oracle_mod.sru_bwd(x["zf"], x["zr"], x["zx"], bf, x["br"], x["gh"], c0=x["c0"],
                           gcl=x["gcl"])
    r = 1.0 / (1.0 + np.exp(-(x["zr"] + x["br"])))
    th = np.tanh(x["c0"])[None]
    assert np.array_equal(g["dzf"], np.zeros_like(g["dzf"]))
    assert np.allclose(g["dzx"], x["gh"] * (1 - r), rtol=0, atol=1e-15)
    dc0 = x["gcl"] + np.sum(x["gh"] * r * (1 - th ** 2), axis=0)
    assert np.allclose(g["dc0"], dc0, rtol=1e-14, atol=1e-14)
    assert np.allclose(g["dzr"], x["gh"] * (th - x["zx"]) * r * (1 - r), rtol=1e-14, atol=1e-15)


def test_forget_gate_open(oracle_mod):
    """b_f = -800: f = 0, so c_t = z_x,t, each step is independent, dL/dc0 = 0
    and dL/dz_x,t = gh_t (1 - r_t) + gh_t r_t (1 - tanh^2 z_x,t) (+ gcl at t = T)."""
    x = case(8, T=5)
    bf = np.full(3, -BIG)
    g = oracle_mod.sru_bwd(x["zf"], x["zr"], x["zx"], bf, x["br"], x["gh"], c0=x["c0"],
                           gcl=x["gcl"])
    r = 1.0 / (1.0 + np.exp(-(x["zr"] + x["br"])))
    th = np.tanh(x["zx"])
    want = x["gh"] * (1 - r) + x["gh"] * r * (1 - th ** 2)
    want[-1] += x["gcl"]
    assert np.allclose(g["dzx"], want, rtol=1e-14, atol=1e-14)
    assert np.array_equal(g["dc0"], np.zeros_like(g["dc0"]))
    assert np.array_equal(g["dzf"], np.zeros_like(g["dzf"]))


def test_bias_gradient_sums_per_feature(oracle_mod):
    """dL/db_f[d] is the sum over batch and time of dL/dz_f at feature d (the
    bias is shared across the batch), and likewise for b_r."""
    x = case(9, T=3, B=4, Dd=2)
    g = oracle_mod.sru_bwd(x["zf"], x["zr"], x["zx"], x["bf"], x["br"], x["gh"], c0=x["c0"])
    assert np.allclose(g["dbf"], g["dzf"].sum(axis=(0, 1)), rtol=1e-13, atol=1e-15)
    assert np.allclose(g["dbr"], g["dzr"].sum(axis=(0, 1)), rtol=1e-13, atol=1e-15)
