"""Diagonal linear-recurrence scan for AMD MI355X (gfx950).

h_t = a_t * h_{t-1} + b_t, element-wise over channels, evaluated as a parallel
prefix scan by hand-written HIP kernels behind the C ABI declared in
include/lrs.h.  This package is the thin Python binding: it marshals torch
device tensors and the current HIP stream into that ABI and nothing more.
"""
# DEER stop rule defaults: eps = 1e-5 and K_max = 5, the example values of the
# DEER page ("cuda-parallel-rnn-training-logt-optimization", engineering section).
DEER_DEFAULT_EPS = 1e-5
DEER_DEFAULT_KMAX = 5

__all__ = ["DEER_DEFAULT_EPS", "DEER_DEFAULT_KMAX"]
