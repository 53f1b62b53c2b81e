"""Diagonal linear-recurrence scan for AMD MI355X (gfx950).

h_t = a_t * h_{t-1} + b_t, element-wise over channels, evaluated as a parallel
prefix scan by hand-written HIP kernels behind the C ABI declared in
include/lrs.h.  The functions exported here come from ``binding`` (a thin
ctypes layer: argument marshalling only, no compute and no fallback).
"""
# DEER stop rule defaults: eps = 1e-5 and K_max = 5, the example values of the
# DEER page ("cuda-parallel-rnn-training-logt-optimization", engineering section).
DEER_DEFAULT_EPS = 1e-5
DEER_DEFAULT_KMAX = 5

_BINDING_NAMES = ("scan_fwd", "scan_bwd", "scan_fwd_bwd", "sru_fwd", "sru_bwd", "deer_solve", "deer_stats",
                  "deer_bwd", "deer_solve_seq", "deer_eps_schedule", "lstm_fwd", "lstm_bwd",
                  "sru_deer_fwd", "rnn_seq", "scan_workspace_bytes", "plan_options",
                  "LrsError", "load")

__all__ = ["DEER_DEFAULT_EPS", "DEER_DEFAULT_KMAX", *_BINDING_NAMES]


def __getattr__(name):
    # the binding imports torch; load it only when a device entry point is used
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
