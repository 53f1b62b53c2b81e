"""fp64 CPU oracle for the diagonal linear recurrence and the layers built on it.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.  It
shares no code with the HIP path.  The arithmetic lives in ``lrs_oracle.c``
(plain sequential loops in double precision); this module only marshals numpy
arrays into it and builds it with gcc.

Every function takes the exact values the device path consumes (fp32 or bf16
values, widened exactly to float64) and returns float64 arrays.

Functions (page citations are in ``lrs_oracle.c``):
  scan_fwd(a, b, h0)            h_t = a_t h_{t-1} + b_t over the last axis
  scan_bwd(a, h, h0, g)         reverse-time adjoint -> (da, db, dh0)
  sru_fwd(zf, zr, zx, bf, br)   SRU layer on [T, B, D] arrays -> (h, c_last)
  sru_bwd(zf, ..., gh, c0, gcl) SRU layer gradients -> dict of six arrays
  lstm_fwd(zf, zi, zc, zo, c0)  LSTM cell-state layer, input-only gates -> (h, c_last)
  lstm_bwd(..., gh, c0, gcl)    its gradients -> dict of five arrays
  sru_nl_seq(zf, ..., vf, c0)   SRU with v_f*c_{t-1} in the forget gate, sequential
  sru_deer(zf, ..., vf, c0)     the same by DEER Newton iterations -> (h, c, iters, deltas)
  rnn_seq(w, u, h0)             sequential h_t = tanh(w h_{t-1} + u_t)
  deer(w, u, h0, ...)           Newton / DEER iterations -> (h, iters, deltas)
  deer_bwd(w, h, g, h0)         adjoint of the RNN at its solution -> (du, dw, dh0)

Parity status: all eleven are pinned by tests/test_oracle_*.py against closed
forms, exact rational brute force, adjoint identities, finite differences and
Newton invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lrs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblrs_oracle.so")
_lib = None

_c_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile lrs_oracle.c with gcc into oracle/liblrs_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.lrs_oracle_scan_fwd.argtypes = [_c_dp, _c_dp, _c_dp, _c_dp, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_scan_bwd.argtypes = [_c_dp, _c_dp, _c_dp, _c_dp, _c_dp, _c_dp, _c_dp,
                                        _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_sru_fwd.argtypes = [_c_dp] * 8 + [_i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_rnn_seq.argtypes = [_c_dp, _c_dp, _c_dp, _c_dp, _i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_deer.argtypes = [_c_dp, _c_dp, _c_dp, _c_dp, _c_dp, _i64, _i64, _i64,
                                    ctypes.c_double, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                    _c_dp, ctypes.c_int]
    lib.lrs_oracle_sru_bwd.argtypes = [_c_dp] * 14 + [_i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_deer_bwd.argtypes = [_c_dp] * 7 + [_i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_lstm_fwd.argtypes = [_c_dp] * 7 + [_i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_lstm_bwd.argtypes = [_c_dp] * 12 + [_i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_sru_nl_seq.argtypes = [_c_dp] * 9 + [_i64, _i64, _i64, ctypes.c_int]
    lib.lrs_oracle_sru_deer.argtypes = [_c_dp] * 10 + [_i64, _i64, _i64, ctypes.c_double,
                                                       ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                                       _c_dp, ctypes.c_int]
    lib.lrs_oracle_sru_nl_seq.restype = ctypes.c_int
    lib.lrs_oracle_sru_deer.restype = ctypes.c_int
    for fn in (lib.lrs_oracle_scan_fwd, lib.lrs_oracle_scan_bwd, lib.lrs_oracle_sru_fwd,
               lib.lrs_oracle_rnn_seq, lib.lrs_oracle_deer, lib.lrs_oracle_sru_bwd,
               lib.lrs_oracle_deer_bwd, lib.lrs_oracle_lstm_fwd, lib.lrs_oracle_lstm_bwd):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(_c_dp)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


def scan_fwd(a, b, h0=None, nthreads: int = 0):
    """h_t = a_t*h_{t-1} + b_t along the last axis.  a, b: [..., T]; h0: [...]."""
    a, b, h0 = _f64(a), _f64(b), _f64(h0)
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    T = a.shape[-1] if a.ndim else 0
    C = a.size // T if T else 0
    if h0 is not None and h0.size != C:
        raise ValueError("h0 must hold one value per channel")
    h = np.empty_like(a)
    _check(_load().lrs_oracle_scan_fwd(_ptr(a), _ptr(b), _ptr(h0), _ptr(h), C, T, nthreads),
           "scan_fwd")
    return h


def scan_bwd(a, h, h0, g, nthreads: int = 0):
    """Adjoint of scan_fwd for L = sum <g, h>.  Returns (da, db, dh0)."""
    a, h, h0, g = _f64(a), _f64(h), _f64(h0), _f64(g)
    if not (a.shape == h.shape == g.shape):
        raise ValueError("a, h, g must have the same shape")
    T = a.shape[-1]
    C = a.size // T if T else 0
    da, db = np.empty_like(a), np.empty_like(a)
    dh0 = np.empty(a.shape[:-1], dtype=np.float64)
    _check(_load().lrs_oracle_scan_bwd(_ptr(a), _ptr(h), _ptr(h0), _ptr(g), _ptr(da), _ptr(db),
                                       _ptr(dh0), C, T, nthreads), "scan_bwd")
    return da, db, dh0


def sru_fwd(zf, zr, zx, bf, br, c0=None, nthreads: int = 0):
    """SRU layer on [T, B, D] pre-activations.  Returns (h [T,B,D], c_last [B,D])."""
    zf, zr, zx, bf, br, c0 = map(_f64, (zf, zr, zx, bf, br, c0))
    if not (zf.shape == zr.shape == zx.shape) or zf.ndim != 3:
        raise ValueError("zf, zr, zx must be [T, B, D]")
    T, B, D = zf.shape
    if bf.shape != (D,) or br.shape != (D,):
        raise ValueError("bf, br must be [D]")
    h = np.empty_like(zf)
    c_last = np.empty((B, D), dtype=np.float64)
    _check(_load().lrs_oracle_sru_fwd(_ptr(zf), _ptr(zr), _ptr(zx), _ptr(bf), _ptr(br), _ptr(c0),
                                      _ptr(h), _ptr(c_last), T, B, D, nthreads), "sru_fwd")
    return h, c_last


def sru_bwd(zf, zr, zx, bf, br, gh, c0=None, gcl=None, nthreads: int = 0):
    """Gradients of the SRU layer for upstream dL/dh = gh [T,B,D] and
    dL/dc_T = gcl [B,D].  Returns dict dzf, dzr, dzx [T,B,D], dbf, dbr [D], dc0 [B,D]."""
    zf, zr, zx, bf, br, gh, c0, gcl = map(_f64, (zf, zr, zx, bf, br, gh, c0, gcl))
    if not (zf.shape == zr.shape == zx.shape == gh.shape) or zf.ndim != 3:
        raise ValueError("zf, zr, zx, gh must be [T, B, D]")
    T, B, D = zf.shape
    if bf.shape != (D,) or br.shape != (D,):
        raise ValueError("bf, br must be [D]")
    out = {k: np.empty_like(zf) for k in ("dzf", "dzr", "dzx")}
    out["dbf"] = np.empty(D)
    out["dbr"] = np.empty(D)
    out["dc0"] = np.empty((B, D))
    _check(_load().lrs_oracle_sru_bwd(_ptr(zf), _ptr(zr), _ptr(zx), _ptr(bf), _ptr(br), _ptr(c0),
                                      _ptr(gh), _ptr(gcl), _ptr(out["dzf"]), _ptr(out["dzr"]),
                                      _ptr(out["dzx"]), _ptr(out["dbf"]), _ptr(out["dbr"]),
                                      _ptr(out["dc0"]), T, B, D, nthreads), "sru_bwd")
    return out


def _lstm_shapes(zs):
    if not all(z.shape == zs[0].shape for z in zs) or zs[0].ndim != 3:
        raise ValueError("zf, zi, zc, zo (and gh) must be [T, B, D] arrays of one shape")
    return zs[0].shape


def lstm_fwd(zf, zi, zc, zo, c0=None, nthreads: int = 0):
    """LSTM cell-state layer with input-only gates on [T, B, D] pre-activations.
    Returns (h [T,B,D], c_last [B,D])."""
    zf, zi, zc, zo, c0 = map(_f64, (zf, zi, zc, zo, c0))
    T, B, D = _lstm_shapes((zf, zi, zc, zo))
    h = np.empty_like(zf)
    c_last = np.empty((B, D))
    _check(_load().lrs_oracle_lstm_fwd(_ptr(zf), _ptr(zi), _ptr(zc), _ptr(zo), _ptr(c0), _ptr(h),
                                       _ptr(c_last), T, B, D, nthreads), "lstm_fwd")
    return h, c_last


def lstm_bwd(zf, zi, zc, zo, gh, c0=None, gcl=None, nthreads: int = 0):
    """Gradients of lstm_fwd for dL/dh = gh [T,B,D] and dL/dc_T = gcl [B,D].
    Returns dict dzf, dzi, dzc, dzo [T,B,D] and dc0 [B,D]."""
    zf, zi, zc, zo, gh, c0, gcl = map(_f64, (zf, zi, zc, zo, gh, c0, gcl))
    T, B, D = _lstm_shapes((zf, zi, zc, zo, gh))
    out = {k: np.empty_like(zf) for k in ("dzf", "dzi", "dzc", "dzo")}
    out["dc0"] = np.empty((B, D))
    _check(_load().lrs_oracle_lstm_bwd(_ptr(zf), _ptr(zi), _ptr(zc), _ptr(zo), _ptr(c0), _ptr(gh),
                                       _ptr(gcl), _ptr(out["dzf"]), _ptr(out["dzi"]),
                                       _ptr(out["dzc"]), _ptr(out["dzo"]), _ptr(out["dc0"]), T, B,
                                       D, nthreads), "lstm_bwd")
    return out


def _sru_nl_args(zf, zr, zx, bf, br, vf, c0):
    zf, zr, zx, bf, br, vf, c0 = map(_f64, (zf, zr, zx, bf, br, vf, c0))
    if not (zf.shape == zr.shape == zx.shape) or zf.ndim != 3:
        raise ValueError("zf, zr, zx must be [T, B, D]")
    D = zf.shape[2]
    if bf.shape != (D,) or br.shape != (D,) or vf.shape != (D,):
        raise ValueError("bf, br, vf must be [D]")
    return zf, zr, zx, bf, br, vf, c0


def sru_nl_seq(zf, zr, zx, bf, br, vf, c0=None, nthreads: int = 0):
    """SRU layer whose forget gate reads v_f * c_{t-1}, by the sequential loop.
    Returns (h [T,B,D], c [T,B,D])."""
    zf, zr, zx, bf, br, vf, c0 = _sru_nl_args(zf, zr, zx, bf, br, vf, c0)
    T, B, D = zf.shape
    h, c = np.empty_like(zf), np.empty_like(zf)
    _check(_load().lrs_oracle_sru_nl_seq(_ptr(zf), _ptr(zr), _ptr(zx), _ptr(bf), _ptr(br),
                                         _ptr(vf), _ptr(c0), _ptr(c), _ptr(h), T, B, D, nthreads),
           "sru_nl_seq")
    return h, c


def sru_deer(zf, zr, zx, bf, br, vf, c0=None, c_init=None, eps: float = 1e-5, k_max: int = 5,
             nthreads: int = 0):
    """The same layer's cell states by DEER Newton iterations.
    Returns (h, c, iters, deltas)."""
    zf, zr, zx, bf, br, vf, c0 = _sru_nl_args(zf, zr, zx, bf, br, vf, c0)
    c_init = _f64(c_init)
    T, B, D = zf.shape
    h, c = np.empty_like(zf), np.empty_like(zf)
    iters = ctypes.c_int(0)
    deltas = np.zeros(max(k_max, 1))
    _check(_load().lrs_oracle_sru_deer(_ptr(zf), _ptr(zr), _ptr(zx), _ptr(bf), _ptr(br), _ptr(vf),
                                       _ptr(c0), _ptr(c_init), _ptr(c), _ptr(h), T, B, D,
                                       float(eps), int(k_max), ctypes.byref(iters), _ptr(deltas),
                                       nthreads), "sru_deer")
    return h, c, iters.value, deltas[: iters.value].copy()


def deer_bwd(w, h, g, h0=None, nthreads: int = 0):
    """Adjoint of h_t = tanh(w h_{t-1} + u_t) at the solution h [B,D,T] for the
    upstream gradient g.  Returns (du [B,D,T], dw [D], dh0 [B,D])."""
    w, h, g, h0 = map(_f64, (w, h, g, h0))
    B, D, T = h.shape
    if g.shape != h.shape or w.shape != (D,):
        raise ValueError("g must match h [B, D, T]; w must be [D]")
    du = np.empty_like(h)
    dw = np.empty(D)
    dh0 = np.empty((B, D))
    _check(_load().lrs_oracle_deer_bwd(_ptr(w), _ptr(h0), _ptr(h), _ptr(g), _ptr(du), _ptr(dw),
                                       _ptr(dh0), B, D, T, nthreads), "deer_bwd")
    return du, dw, dh0


def rnn_seq(w, u, h0=None, nthreads: int = 0):
    """Sequential h_t = tanh(w_d h_{t-1} + u_t); u: [B, D, T], w: [D]."""
    w, u, h0 = _f64(w), _f64(u), _f64(h0)
    B, D, T = u.shape
    if w.shape != (D,):
        raise ValueError("w must be [D]")
    h = np.empty_like(u)
    _check(_load().lrs_oracle_rnn_seq(_ptr(w), _ptr(u), _ptr(h0), _ptr(h), B, D, T, nthreads),
           "rnn_seq")
    return h


def deer(w, u, h0=None, h_init=None, eps: float = 1e-5, k_max: int = 5, nthreads: int = 0):
    """DEER Newton iterations for h_t = tanh(w h_{t-1} + u_t).

    Returns (h, iters, deltas) with deltas[i] = max |y^(i+1) - y^(i)|."""
    w, u, h0, h_init = _f64(w), _f64(u), _f64(h0), _f64(h_init)
    B, D, T = u.shape
    if w.shape != (D,):
        raise ValueError("w must be [D]")
    h = np.empty_like(u)
    iters = ctypes.c_int(0)
    deltas = np.zeros(max(k_max, 1), dtype=np.float64)
    _check(_load().lrs_oracle_deer(_ptr(w), _ptr(u), _ptr(h0), _ptr(h_init), _ptr(h), B, D, T,
                                   float(eps), int(k_max), ctypes.byref(iters), _ptr(deltas),
                                   nthreads), "deer")
    return h, iters.value, deltas[: iters.value].copy()
