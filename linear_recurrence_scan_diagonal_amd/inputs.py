"""Seeded synthetic inputs for the scan, SRU, LSTM and DEER workloads.

This module only draws random numbers and converts number formats; it holds
none of the method's arithmetic, so both the device path and the CPU oracle
can be fed from it.

Recipe (the same everywhere):
  * every per-time-step array is drawn channel by channel; channel ``c`` of
    array ``tag`` uses its own PCG64 stream seeded with
    ``SeedSequence([seed, tag, c])`` and draws its T values in time order, in
    float64;
  * per-channel or per-feature parameters ([B, D] or [D]) use the stream
    ``SeedSequence([seed, tag])`` and are drawn in C order;
  * each float64 draw is rounded once, to nearest-even, to the I/O type
    (fp32 or bf16).  Those rounded values are the canonical inputs: the device
    receives them and the oracle receives them widened exactly to float64.
  * ``normal(mu, s)`` takes the standard deviation ``s``; ``uniform(lo, hi)``
    draws from [lo, hi).

Arrays above 2^31 elements (the size-limit tests) are drawn on the device
instead, by ``device_draw``: torch's Philox generator seeded with
``seed``, one call per array, in fp32 (``uniform(lo, hi)`` as
lo + (hi - lo) * U[0, 1), ``normal(mu, s)`` as mu + s * N(0, 1), each rounded
to fp32), optionally rounded once more to bf16.  Those device values are the
canonical inputs of such a test; the oracle receives host copies of the parts
it checks, widened exactly to float64.

Array tags: a=1, b=2, h0=3, g=4, zf=5, zr=6, zx=7, bias_f=8, bias_r=9, w=10,
u=11, h_init=12, gh=13, gcl=14, zi=15, zc=16, zo=17, vf=18.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TAGS = {"a": 1, "b": 2, "h0": 3, "g": 4, "zf": 5, "zr": 6, "zx": 7, "bias_f": 8,
        "bias_r": 9, "w": 10, "u": 11, "h_init": 12, "gh": 13, "gcl": 14, "zi": 15, "zc": 16,
        "zo": 17, "vf": 18}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _draw(rng: np.random.Generator, dist, n: int) -> np.ndarray:
    kind, p, q = dist
    if kind == "uniform":
        return rng.uniform(p, q, n)
    if kind == "normal":
        return rng.normal(p, q, n)
    if kind == "const":
        return np.full(n, float(p))
    raise ValueError(f"unknown distribution {kind!r}")


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def series(seed: int, tag: str, dist, channels, T: int, dtype=np.float64) -> np.ndarray:
    """[len(channels), T] per-channel streams in time order, drawn in float64.

    dtype=np.float32 rounds each row once to fp32 as it is drawn (same values
    as to_f32(series(...)), without holding the float64 array)."""
    channels = np.asarray(list(channels), dtype=np.int64)
    out = np.empty((channels.size, T), dtype=dtype)
    t = TAGS[tag]

    def fill(lo, hi):
        for i in range(lo, hi):
            out[i] = _draw(_rng(seed, t, int(channels[i])), dist, T)  # one rounding on assignment

    n = channels.size
    step = max(1, (n + _workers() * 4 - 1) // (_workers() * 4))
    if n * T < (1 << 16):
        fill(0, n)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(lambda lo: fill(lo, min(n, lo + step)), range(0, n, step)))
    return out


def params(seed: int, tag: str, dist, shape) -> np.ndarray:
    """float64 array of the given shape from one stream, C order."""
    n = int(np.prod(shape)) if len(shape) else 1
    return _draw(_rng(seed, TAGS[tag]), dist, n).reshape(shape)


# ----- number formats -------------------------------------------------------

def to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to fp32, nearest-even."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 once to bfloat16 (nearest-even); return the uint16 bit patterns.

    Works on the float64 bit pattern directly so there is a single rounding.
    Values must lie inside the normal bf16 range (true for every recipe here)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding helper expects finite values")
    bits = x.view(np.uint64)
    # bf16 keeps 7 of float64's 52 fraction bits: round at bit 45.
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    as_f32 = rounded.view(np.float64).astype(np.float32)  # exact: <= 8 significant bits
    if not np.all(np.isfinite(as_f32)):
        raise ValueError("value outside the bf16 range")
    return (as_f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


# ----- the workloads ---------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "scan", "sru", "sru_deer", "lstm" or "deer"
    B: int
    D: int
    T: int
    seed: int
    dists: dict = field(default_factory=dict)
    desc: str = ""
    io: str = "f32"           # element type of the scan arrays: "f32" or "bf16"

    @property
    def C(self) -> int:
        return self.B * self.D

    @property
    def N(self) -> int:
        return self.B * self.D * self.T


WORKLOADS = {
    # forward scan only, fp32, [B, D, T]
    "scan_fwd_small": Workload(
        "scan_fwd_small", "scan", 1, 64, 1024, 1001,
        {"a": ("uniform", 0.5, 1.0), "b": ("normal", 0.0, 1.0), "h0": ("const", 0.0, 0.0)},
        "forward linear scan, fp32, B=1 D=64 T=1024, a~U(0.5,1), b~N(0,1), h0=0"),
    # forward + backward scan, fp32
    "scan_fwd_bwd": Workload(
        "scan_fwd_bwd", "scan", 8, 512, 4096, 1002,
        {"a": ("uniform", 0.8, 0.999), "b": ("normal", 0.0, 1.0), "h0": ("normal", 0.0, 1.0),
         "g": ("normal", 0.0, 1.0)},
        "forward+backward linear scan, fp32, B=8 D=512 T=4096, a~U(0.8,0.999), b~N(0,1), "
        "h0~N(0,1), dL/dh~N(0,1)"),
    # the same forward + backward scan as one lrs_scan_fwd_bwd call (same inputs)
    "scan_fused": Workload(
        "scan_fused", "scan", 8, 512, 4096, 1002,
        {"a": ("uniform", 0.8, 0.999), "b": ("normal", 0.0, 1.0), "h0": ("normal", 0.0, 1.0),
         "g": ("normal", 0.0, 1.0)},
        "forward+backward linear scan in one call, fp32, B=8 D=512 T=4096, inputs as "
        "scan_fwd_bwd"),
    # forward + backward scan of many short channels (sequential kernels)
    "scan_short": Workload(
        "scan_short", "scan", 256, 2048, 32, 1009,
        {"a": ("uniform", 0.8, 0.999), "b": ("normal", 0.0, 1.0), "h0": ("normal", 0.0, 1.0),
         "g": ("normal", 0.0, 1.0)},
        "forward+backward linear scan of short channels, fp32, B=256 D=2048 T=32, "
        "distributions as scan_fwd_bwd"),
    # SRU layer forward, bf16 I/O, fp32 state, [T, B, D]
    "sru_fwd": Workload(
        "sru_fwd", "sru", 32, 1024, 2048, 1003,
        {"zf": ("normal", 0.0, 1.0), "zr": ("normal", 0.0, 1.0), "zx": ("normal", 0.0, 1.0),
         "bias_f": ("normal", -1.0, 0.1), "bias_r": ("normal", -1.0, 0.1)},
        "SRU forward, bf16 I/O fp32 state, B=32 D=1024 T=2048, z~N(0,1), b_f,b_r~N(-1,0.1), c0=0"),
    # SRU forward (saving the cell states) and backward at the SRU shape; the
    # upstream gradient dL/dh ~ N(0,1) as for the scan workloads
    "sru_fwd_bwd": Workload(
        "sru_fwd_bwd", "sru", 32, 1024, 2048, 1006,
        {"zf": ("normal", 0.0, 1.0), "zr": ("normal", 0.0, 1.0), "zx": ("normal", 0.0, 1.0),
         "bias_f": ("normal", -1.0, 0.1), "bias_r": ("normal", -1.0, 0.1),
         "gh": ("normal", 0.0, 1.0)},
        "SRU forward + backward, bf16 I/O fp32 state, B=32 D=1024 T=2048, z~N(0,1), "
        "b_f,b_r~N(-1,0.1), c0=0, dL/dh~N(0,1)"),
    # SRU whose forget gate reads v_f * c_{t-1}, solved by DEER, at the SRU shape
    "sru_deer": Workload(
        "sru_deer", "sru_deer", 32, 1024, 2048, 1010,
        {"zf": ("normal", 0.0, 1.0), "zr": ("normal", 0.0, 1.0), "zx": ("normal", 0.0, 1.0),
         "bias_f": ("normal", -1.0, 0.1), "bias_r": ("normal", -1.0, 0.1),
         "vf": ("uniform", -0.25, 0.25)},
        "SRU with v_f*c_{t-1} in the forget gate by DEER, bf16 I/O fp32 state, B=32 D=1024 "
        "T=2048, z~N(0,1), b_f,b_r~N(-1,0.1), v_f~U(-0.25,0.25), c0=0, c_init=0, eps=1e-5, "
        "K_max=5"),
    # LSTM cell-state layer with input-only gates, forward (saving the cell
    # states) and backward, at the SRU shape
    "lstm_fwd_bwd": Workload(
        "lstm_fwd_bwd", "lstm", 32, 1024, 2048, 1008,
        {"zf": ("normal", 0.0, 1.0), "zi": ("normal", 0.0, 1.0), "zc": ("normal", 0.0, 1.0),
         "zo": ("normal", 0.0, 1.0), "gh": ("normal", 0.0, 1.0)},
        "LSTM cell-state layer (input-only gates) forward + backward, bf16 I/O fp32 state, "
        "B=32 D=1024 T=2048, z_f,z_i,z_c,z_o~N(0,1), c0=0, dL/dh~N(0,1)"),
    # the forward + backward scan with bf16 arrays (fp32 state): scan_fwd_bwd's
    # shape and distributions, a, b and dL/dh rounded to bf16
    "scan_fwd_bwd_bf16": Workload(
        "scan_fwd_bwd_bf16", "scan", 8, 512, 4096, 1011,
        {"a": ("uniform", 0.8, 0.999), "b": ("normal", 0.0, 1.0), "h0": ("normal", 0.0, 1.0),
         "g": ("normal", 0.0, 1.0)},
        "forward+backward linear scan, bf16 arrays with fp32 state, B=8 D=512 T=4096, "
        "a~U(0.8,0.999), b~N(0,1), h0~N(0,1), dL/dh~N(0,1) (a, b, dL/dh rounded to bf16)",
        io="bf16"),
    # very long forward + backward scan, fp32
    "scan_long": Workload(
        "scan_long", "scan", 2, 256, 1 << 20, 1004,
        {"a": ("uniform", 0.9, 0.9999), "b": ("normal", 0.0, 0.1), "h0": ("const", 0.0, 0.0),
         "g": ("normal", 0.0, 1.0)},
        "long forward+backward linear scan, fp32, B=2 D=256 T=2^20, a~U(0.9,0.9999), "
        "b~N(0,0.1), h0=0, dL/dh~N(0,1)"),
    # the long scan with bf16 arrays (fp32 state)
    "scan_long_bf16": Workload(
        "scan_long_bf16", "scan", 2, 256, 1 << 20, 1012,
        {"a": ("uniform", 0.9, 0.9999), "b": ("normal", 0.0, 0.1), "h0": ("const", 0.0, 0.0),
         "g": ("normal", 0.0, 1.0)},
        "long forward+backward linear scan, bf16 arrays with fp32 state, B=2 D=256 T=2^20, "
        "a~U(0.9,0.9999), b~N(0,0.1), h0=0, dL/dh~N(0,1) (a, b, dL/dh rounded to bf16)",
        io="bf16"),
    # DEER Newton solve of h_t = tanh(w h_{t-1} + u_t)
    "deer": Workload(
        "deer", "deer", 16, 512, 8192, 1005,
        {"w": ("uniform", -0.9, 0.9), "u": ("normal", 0.0, 1.0), "h0": ("const", 0.0, 0.0)},
        "DEER Newton solve, fp32, B=16 D=512 T=8192, w~U(-0.9,0.9) per feature, u~N(0,1), "
        "h0=0, h_init=0, eps=1e-5, K_max=5"),
    # the DEER solve followed by the backward at its solution, dL/dh ~ N(0,1)
    "deer_fwd_bwd": Workload(
        "deer_fwd_bwd", "deer", 16, 512, 8192, 1007,
        {"w": ("uniform", -0.9, 0.9), "u": ("normal", 0.0, 1.0), "h0": ("const", 0.0, 0.0),
         "g": ("normal", 0.0, 1.0)},
        "DEER solve + backward, fp32, B=16 D=512 T=8192, as the DEER workload plus "
        "dL/dh~N(0,1)"),
}


def scaled(w: Workload, B=None, D=None, T=None, seed=None) -> Workload:
    """Same distributions, other sizes (for small parity cases)."""
    return Workload(w.name, w.kind, B or w.B, D or w.D, T or w.T,
                    w.seed if seed is None else seed, dict(w.dists), w.desc, w.io)


def scan_inputs(w: Workload, channels=None, with_grad: bool = True) -> dict:
    """fp32 arrays for the scan workloads, [len(channels), T] (channel-major).

    channels defaults to all B*D channels; h0 is returned as [len(channels)]."""
    ch = np.arange(w.C) if channels is None else np.asarray(channels)
    f32 = np.float32
    out = {"a": series(w.seed, "a", w.dists["a"], ch, w.T, f32),
           "b": series(w.seed, "b", w.dists["b"], ch, w.T, f32)}
    h0 = to_f32(params(w.seed, "h0", w.dists.get("h0", ("const", 0, 0)), (w.C,)))
    out["h0"] = h0[ch]
    if with_grad and "g" in w.dists:
        out["g"] = series(w.seed, "g", w.dists["g"], ch, w.T, f32)
    return out


def scan_inputs_bf16(w: Workload, channels=None, with_grad: bool = True, batch: int = 64) -> dict:
    """bf16 bit patterns (uint16) of a, b and g, [len(channels), T] channel-major,
    each value rounded once from its float64 draw; h0 fp32 [len(channels)].
    Drawn in batches of channels so the float64 rows are never all held."""
    ch = np.arange(w.C) if channels is None else np.asarray(channels)
    tags = ("a", "b", "g") if with_grad and "g" in w.dists else ("a", "b")
    out = {k: np.empty((ch.size, w.T), dtype=np.uint16) for k in tags}
    for lo in range(0, ch.size, batch):
        part = ch[lo:lo + batch]
        for k in tags:
            out[k][lo:lo + part.size] = to_bf16_bits(series(w.seed, k, w.dists[k], part, w.T))
    h0 = to_f32(params(w.seed, "h0", w.dists.get("h0", ("const", 0, 0)), (w.C,)))
    out["h0"] = h0[ch]
    return out


def sru_inputs(w: Workload) -> dict:
    """bf16 bit patterns of zf, zr, zx as [T, B, D] uint16 arrays, fp32 biases [D]."""
    ch = np.arange(w.C)
    out = {}
    for k in ("zf", "zr", "zx"):
        per_channel = to_bf16_bits(series(w.seed, k, w.dists[k], ch, w.T))  # [C, T]
        out[k] = np.ascontiguousarray(per_channel.T).reshape(w.T, w.B, w.D)
    out["bias_f"] = to_f32(params(w.seed, "bias_f", w.dists["bias_f"], (w.D,)))
    out["bias_r"] = to_f32(params(w.seed, "bias_r", w.dists["bias_r"], (w.D,)))
    return out


def sru_vf(w: Workload) -> np.ndarray:
    """fp32 v_f [D] (the forget gate's weight on c_{t-1})."""
    return to_f32(params(w.seed, "vf", w.dists["vf"], (w.D,)))


def lstm_inputs(w: Workload) -> dict:
    """bf16 bit patterns of the pre-activations zf, zi, zc, zo as [T, B, D] uint16."""
    ch = np.arange(w.C)
    out = {}
    for k in ("zf", "zi", "zc", "zo"):
        per_channel = to_bf16_bits(series(w.seed, k, w.dists[k], ch, w.T))  # [C, T]
        out[k] = np.ascontiguousarray(per_channel.T).reshape(w.T, w.B, w.D)
    return out


def sru_grad_inputs(w: Workload, with_gcl: bool = False) -> dict:
    """Upstream gradients for the SRU (and LSTM) backward: dL/dh as bf16 bit patterns
    [T, B, D] uint16 (drawn like the pre-activations), and optionally
    dL/dc_T as fp32 [B, D] from N(0,1)."""
    ch = np.arange(w.C)
    dist = w.dists.get("gh", ("normal", 0.0, 1.0))
    per_channel = to_bf16_bits(series(w.seed, "gh", dist, ch, w.T))
    out = {"gh": np.ascontiguousarray(per_channel.T).reshape(w.T, w.B, w.D)}
    if with_gcl:
        out["gcl"] = to_f32(params(w.seed, "gcl", ("normal", 0.0, 1.0), (w.C,))).reshape(w.B, w.D)
    return out


def deer_inputs(w: Workload, channels=None) -> dict:
    """fp32 w [D], u [len(channels), T] (channel-major), h0 [len(channels)]."""
    ch = np.arange(w.C) if channels is None else np.asarray(channels)
    out = {"w": to_f32(params(w.seed, "w", w.dists["w"], (w.D,))),
           "u": series(w.seed, "u", w.dists["u"], ch, w.T, np.float32)}
    h0 = to_f32(params(w.seed, "h0", w.dists.get("h0", ("const", 0, 0)), (w.C,)))
    out["h0"] = h0[ch]
    return out


def device_draw(seed: int, dist, shape, device, bf16: bool = False):
    """Seeded draw of a (possibly > 2^31-element) array on the device; see the
    module docstring.  dist as for ``series`` (uniform / normal / const)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    kind, p, q = dist
    if kind == "uniform":
        x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(float(q) - float(p)).add_(float(p))
    elif kind == "normal":
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(float(q)).add_(float(p))
    elif kind == "const":
        x = torch.full(shape, float(p), device=device, dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {kind!r}")
    return x.to(torch.bfloat16) if bf16 else x
