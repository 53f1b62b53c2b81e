"""The oracle's pins are not vacuous: copies of lrs_oracle.c with one plausible
mistake planted (a dropped term, a wrong sign, a shifted time index, a
missing factor of the Jacobian) are compiled on the CPU and each must fail at
least one pin of the function it breaks, while the unmodified oracle passes
them all (the other test modules)."""
import inspect
import itertools
import os
import subprocess

import pytest

import oracle
import test_oracle_deer_bwd
import test_oracle_lstm
import test_oracle_scan
import test_oracle_sru_bwd
import test_oracle_sru_nl

# (what is planted, original text, mutated text, which occurrence, pin module)
MUTATIONS = [
    ("scan backward: coefficient of the same step instead of the next",
     "double next = (t + 1 < T) ? ac[t + 1] * lam : 0.0;",
     "double next = (t + 1 < T) ? ac[t] * lam : 0.0;", 0, test_oracle_scan),
    ("SRU backward: sign of (c_{t-1} - z_x) flipped",
     "dzf[i] = gc * (cprev - zx[i]) * f * (1.0 - f);",
     "dzf[i] = gc * (zx[i] - cprev) * f * (1.0 - f);", 0, test_oracle_sru_bwd),
    ("LSTM forward: input gate dropped",
     "c = f * c + i * g;", "c = f * c + g;", 0, test_oracle_lstm),
    ("LSTM backward: candidate factor dropped from dz_i",
     "dzi[k] = gc * g * i * (1.0 - i);", "dzi[k] = gc * i * (1.0 - i);", 0, test_oracle_lstm),
    ("LSTM backward: c_t used where c_{t-1} belongs",
     "const double cprev = t > 0 ? c[t - 1] : (c0 ? c0[ch] : 0.0);",
     "const double cprev = t > 0 ? c[t] : (c0 ? c0[ch] : 0.0);", 1, test_oracle_lstm),
    ("non-linear SRU: forget gate reads z_x instead of c_{t-1}",
     "vf[d] * state", "vf[d] * zx[i]", 0, test_oracle_sru_nl),
    ("SRU by DEER: Jacobian loses its (1 - f) factor",
     "* f * (1.0 - f) * vf[d];", "* f * vf[d];", 0, test_oracle_sru_nl),
    ("DEER backward: derivative of the step itself instead of the next",
     "wd * s_next * lam_next : 0.0);\n            const double hprev",
     "wd * s * lam_next : 0.0);\n            const double hprev", 0, test_oracle_deer_bwd),
]


def replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


def pin_calls(module):
    """Every test function of a pin module with each of its parameter sets."""
    for name, fn in sorted(vars(module).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            names = [s.strip() for s in m.args[0].split(",")] if isinstance(m.args[0], str) \
                else list(m.args[0])
            vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(names, v)) for v in vals])
        for combo in itertools.product(*grids) if grids else [()]:
            kwargs = {}
            for d in combo:
                kwargs.update(d)
            yield name, fn, kwargs


@pytest.mark.parametrize("what,old,new,nth,module", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, monkeypatch, what, old, new, nth, module):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "lrs_oracle.c")).read()
    assert old in src, f"mutation site not found: {old}"
    bad_src = tmp_path / "lrs_oracle_mut.c"
    bad_src.write_text(replace_nth(src, old, new, nth))
    lib = tmp_path / "liblrs_oracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(lib), str(bad_src), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_LIB_PATH", str(lib))
    monkeypatch.setattr(oracle, "_lib", None)
    failed = []
    for name, fn, kwargs in pin_calls(module):
        args = {"oracle_mod": oracle} if "oracle_mod" in inspect.signature(fn).parameters else {}
        try:
            fn(**args, **kwargs)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.append(name)
    monkeypatch.setattr(oracle, "_lib", None)
    assert failed, f"no pin of {module.__name__} caught: {what}"
