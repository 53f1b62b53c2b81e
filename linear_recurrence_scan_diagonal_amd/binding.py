"""ctypes binding of liblrs.so (include/lrs.h), one Python function per entry point.

Argument marshalling only: shapes and dtypes are checked, outputs and
workspaces are allocated as torch device tensors, and the raw pointers plus the
current HIP stream are handed to the C ABI.  Every step of the computation
runs in the library's HIP kernels; there is no fallback of any kind, and a
missing library raises at once.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrs.so")

LRS_OK, LRS_ERR_INVALID_ARG, LRS_ERR_UNSUPPORTED, LRS_ERR_WORKSPACE, LRS_ERR_HIP, \
    LRS_ERR_NONFINITE = range(6)
LAYOUTS = {"bdt": 0, "tbd": 1}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}

EXPORTS = ("lrs_status_string", "lrs_version", "lrs_scan_workspace_bytes", "lrs_scan_fwd",
           "lrs_scan_bwd", "lrs_sru_workspace_bytes", "lrs_sru_fwd", "lrs_deer_workspace_bytes",
           "lrs_deer_solve", "lrs_deer_stats", "lrs_sru_bwd_workspace_bytes", "lrs_sru_bwd",
           "lrs_deer_bwd_workspace_bytes", "lrs_deer_bwd", "lrs_lstm_workspace_bytes",
           "lrs_lstm_fwd", "lrs_lstm_bwd", "lrs_scan_fwd_bwd", "lrs_sru_deer_workspace_bytes",
           "lrs_sru_deer_fwd", "lrs_deer_seq_workspace_bytes", "lrs_deer_solve_seq",
           "lrs_rnn_seq")

# entry points that have an _ex variant taking lrs_options
_EX_BASES = ("lrs_scan_fwd", "lrs_scan_bwd", "lrs_scan_fwd_bwd", "lrs_sru_fwd", "lrs_sru_deer_fwd",
             "lrs_deer_solve", "lrs_deer_solve_seq", "lrs_lstm_fwd")
EXPORTS = EXPORTS + tuple(n + "_ex" for n in _EX_BASES) + ("lrs_options_default",
                                                            "lrs_deer_eps_schedule",
                                                            "lrs_scan_fwd_bwd_noalloc")


class LrsOptions(ctypes.Structure):
    """lrs_options (include/lrs.h): explicit plan choices, -1 = the default."""
    _fields_ = [("serial_fwd_max_t", ctypes.c_int64), ("serial_bwd_max_t", ctypes.c_int64),
                ("packed_max_t", ctypes.c_int64), ("persist_min_blocks", ctypes.c_int64),
                ("deer_fuse", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_plan = threading.local()


@contextlib.contextmanager
def plan_options(**fields):
    """Inside the block, calls that accept `options` and get none pass these
    lrs_options fields (merged over those of an enclosing block) to the
    library's _ex entry point.  The choice still travels as an explicit
    argument of every call; the library itself keeps no state."""
    prev = getattr(_plan, "opts", None)
    merged = dict(prev or {})
    merged.update(fields)
    _plan.opts = merged
    try:
        yield
    finally:
        _plan.opts = prev


def _opts(options):
    """None, or a dict of lrs_options fields (others keep the defaults), ->
    the pointer argument of an _ex entry point."""
    if options is None:
        options = getattr(_plan, "opts", None)
    if options is None:
        return None
    o = LrsOptions()
    load().lrs_options_default(ctypes.byref(o))
    for k, v in dict(options).items():
        if k not in ("serial_fwd_max_t", "serial_bwd_max_t", "packed_max_t",
                     "persist_min_blocks", "deer_fuse"):
            raise ValueError(f"unknown option {k!r}")
        setattr(o, k, int(v))
    return ctypes.byref(o)


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t


class LrsError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = load().lrs_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{where}: {msg}")


def load():
    """Load liblrs.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                           "g.build()'` first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.lrs_status_string.argtypes = [_int]
    lib.lrs_status_string.restype = ctypes.c_char_p
    lib.lrs_version.argtypes = []
    lib.lrs_version.restype = _int
    lib.lrs_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int]
    lib.lrs_scan_workspace_bytes.restype = _sz
    lib.lrs_scan_fwd.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]
    lib.lrs_scan_fwd.restype = _int
    lib.lrs_scan_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                 _vp, _sz, _vp]
    lib.lrs_scan_bwd.restype = _int
    lib.lrs_scan_fwd_bwd.argtypes = [_vp] * 8 + [_i64, _i64, _i64, _int, _int, _vp, _sz, _vp]
    lib.lrs_scan_fwd_bwd.restype = _int
    lib.lrs_sru_workspace_bytes.argtypes = [_i64, _i64, _i64]
    lib.lrs_sru_workspace_bytes.restype = _sz
    lib.lrs_sru_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int,
                                _vp, _sz, _vp]
    lib.lrs_sru_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64]
    lib.lrs_sru_bwd_workspace_bytes.restype = _sz
    lib.lrs_sru_bwd.argtypes = [_vp] * 15 + [_i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.lrs_sru_bwd.restype = _int
    lib.lrs_sru_fwd.restype = _int
    lib.lrs_deer_seq_workspace_bytes.argtypes = [_i64, _i64, _i64, _int]
    lib.lrs_deer_seq_workspace_bytes.restype = _sz
    lib.lrs_deer_solve_seq.argtypes = [_vp] * 5 + [_i64, _i64, _i64, ctypes.c_float, _int, _vp,
                                                   _vp, _vp, _sz, _vp]
    lib.lrs_deer_solve_seq.restype = _int
    lib.lrs_sru_deer_workspace_bytes.argtypes = [_i64, _i64, _i64, _int]
    lib.lrs_sru_deer_workspace_bytes.restype = _sz
    lib.lrs_sru_deer_fwd.argtypes = [_vp] * 11 + [_i64, _i64, _i64, _int, ctypes.c_float, _int,
                                                  _vp, _vp, _vp, _vp, _sz, _vp]
    lib.lrs_sru_deer_fwd.restype = _int
    lib.lrs_lstm_workspace_bytes.argtypes = [_i64, _i64, _i64]
    lib.lrs_lstm_workspace_bytes.restype = _sz
    lib.lrs_lstm_fwd.argtypes = [_vp] * 8 + [_i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.lrs_lstm_fwd.restype = _int
    lib.lrs_lstm_bwd.argtypes = [_vp] * 13 + [_i64, _i64, _i64, _int, _vp, _sz, _vp]
    lib.lrs_lstm_bwd.restype = _int
    lib.lrs_deer_workspace_bytes.argtypes = [_i64, _i64, _i64, _int]
    lib.lrs_deer_workspace_bytes.restype = _sz
    lib.lrs_deer_solve.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_float, _int,
                                   ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_float),
                                   ctypes.POINTER(_int), _vp, _sz, _vp]
    lib.lrs_deer_solve.restype = _int
    lib.lrs_deer_stats.argtypes = [_vp, _sz, _int, ctypes.POINTER(_int),
                                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_int), _vp]
    lib.lrs_deer_stats.restype = _int
    lib.lrs_deer_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64]
    lib.lrs_deer_bwd_workspace_bytes.restype = _sz
    lib.lrs_deer_bwd.argtypes = [_vp] * 7 + [_i64, _i64, _i64, _vp, _sz, _vp]
    lib.lrs_deer_bwd.restype = _int
    lib.lrs_rnn_seq.argtypes = [_vp] * 4 + [_i64, _i64, _i64, _vp]
    lib.lrs_rnn_seq.restype = _int
    lib.lrs_options_default.argtypes = [ctypes.POINTER(LrsOptions)]
    lib.lrs_options_default.restype = None
    for name in _EX_BASES:
        base = getattr(lib, name)
        ex = getattr(lib, name + "_ex")
        ex.argtypes = list(base.argtypes) + [ctypes.POINTER(LrsOptions)]
        ex.restype = _int
    lib.lrs_scan_fwd_bwd_noalloc.argtypes = [_vp] * 8 + [_i64, _i64, _i64, _int, _int, _vp]
    lib.lrs_scan_fwd_bwd_noalloc.restype = _int
    lib.lrs_deer_eps_schedule.argtypes = [_i64, _i64, ctypes.c_float, ctypes.c_float]
    lib.lrs_deer_eps_schedule.restype = ctypes.c_float
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check_dev(name, t, dtype, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _dims(x: torch.Tensor, layout: str):
    if x.dim() != 3:
        raise ValueError("expected a 3-d tensor")
    if layout == "bdt":
        B, D, T = x.shape
    elif layout == "tbd":
        T, B, D = x.shape
    else:
        raise ValueError(f"layout must be 'bdt' or 'tbd', got {layout!r}")
    return int(B), int(D), int(T)


def _call(rc: int, where: str):
    if rc != LRS_OK:
        raise LrsError(rc, where)


def scan_workspace_bytes(B, D, T, layout="bdt", dtype=torch.float32) -> int:
    return int(load().lrs_scan_workspace_bytes(B, D, T, LAYOUTS[layout], DTYPES[dtype]))


def scan_fwd(a, b, h0=None, layout: str = "bdt", out=None, workspace=None, options=None):
    """h_t = a_t*h_{t-1} + b_t.  a, b: [B,D,T] ('bdt') or [T,B,D] ('tbd'); h0: [B,D]."""
    lib = load()
    B, D, T = _dims(a, layout)
    _check_dev("a", a, a.dtype, a.shape)
    _check_dev("b", b, a.dtype, a.shape)
    _check_dev("h0", h0, torch.float32, (B, D))
    h = torch.empty_like(a) if out is None else out
    _check_dev("out", h, a.dtype, a.shape)
    nbytes = lib.lrs_scan_workspace_bytes(B, D, T, LAYOUTS[layout], DTYPES[a.dtype])
    ws = _workspace(nbytes, a.device, workspace)
    _call(lib.lrs_scan_fwd_ex(_ptr(a), _ptr(b), _ptr(h0), _ptr(h), B, D, T, LAYOUTS[layout],
                           DTYPES[a.dtype], _ptr(ws), nbytes, _stream(a.device), _opts(options)), "lrs_scan_fwd")
    return h


def scan_bwd(a, h, grad_h, h0=None, layout: str = "bdt", need_grad_h0: bool = True,
             grad_a=None, grad_b=None, grad_h0=None, workspace=None, options=None):
    """Reverse-time adjoint.  Returns (grad_a, grad_b, grad_h0 or None).
    grad_b may be passed as grad_h itself (in-place)."""
    lib = load()
    B, D, T = _dims(a, layout)
    for name, t in (("a", a), ("h", h), ("grad_h", grad_h)):
        _check_dev(name, t, a.dtype, a.shape)
    _check_dev("h0", h0, torch.float32, (B, D))
    ga = torch.empty_like(a) if grad_a is None else grad_a
    gb = torch.empty_like(a) if grad_b is None else grad_b
    gh0 = None
    if need_grad_h0:
        gh0 = torch.empty((B, D), dtype=torch.float32, device=a.device) if grad_h0 is None else grad_h0
    _check_dev("grad_a", ga, a.dtype, a.shape)
    _check_dev("grad_b", gb, a.dtype, a.shape)
    _check_dev("grad_h0", gh0, torch.float32, (B, D))
    nbytes = lib.lrs_scan_workspace_bytes(B, D, T, LAYOUTS[layout], DTYPES[a.dtype])
    ws = _workspace(nbytes, a.device, workspace)
    _call(lib.lrs_scan_bwd_ex(_ptr(a), _ptr(h), _ptr(h0), _ptr(grad_h), _ptr(ga), _ptr(gb), _ptr(gh0),
                           B, D, T, LAYOUTS[layout], DTYPES[a.dtype], _ptr(ws), nbytes,
                           _stream(a.device), _opts(options)), "lrs_scan_bwd")
    return ga, gb, gh0


def scan_fwd_bwd(a, b, grad_h, h0=None, layout: str = "bdt", want_h: bool = True,
                 need_grad_h0: bool = True, out=None, workspace=None, options=None):
    """scan_fwd then scan_bwd in one call (one kernel for [B,D,T] channels of
    up to 8192 steps).  Returns (h or None, grad_a, grad_b, grad_h0 or None).
    want_h=False skips writing h (only where one kernel does both passes).
    out: optional (h, grad_a, grad_b, grad_h0) tensors; grad_b may be grad_h."""
    lib = load()
    B, D, T = _dims(a, layout)
    for name, t in (("a", a), ("b", b), ("grad_h", grad_h)):
        _check_dev(name, t, a.dtype, a.shape)
    _check_dev("h0", h0, torch.float32, (B, D))
    if out is None:
        out = (torch.empty_like(a) if want_h else None, torch.empty_like(a), torch.empty_like(a),
               torch.empty((B, D), dtype=torch.float32, device=a.device) if need_grad_h0 else None)
    h, ga, gb, gh0 = out
    for name, t in (("h", h), ("grad_a", ga), ("grad_b", gb)):
        _check_dev(name, t, a.dtype, a.shape)
    _check_dev("grad_h0", gh0, torch.float32, (B, D))
    nbytes = lib.lrs_scan_workspace_bytes(B, D, T, LAYOUTS[layout], DTYPES[a.dtype])
    ws = _workspace(nbytes, a.device, workspace)
    _call(lib.lrs_scan_fwd_bwd_ex(_ptr(a), _ptr(b), _ptr(h0), _ptr(grad_h), _ptr(h), _ptr(ga),
                               _ptr(gb), _ptr(gh0), B, D, T, LAYOUTS[layout], DTYPES[a.dtype],
                               _ptr(ws), nbytes, _stream(a.device), _opts(options)), "lrs_scan_fwd_bwd")
    return h, ga, gb, gh0


def sru_fwd(z_f, z_r, z_x, bias_f, bias_r, c0=None, want_c_last: bool = False, out=None,
            workspace=None, c_states=None, options=None):
    """Fused SRU layer on [T,B,D] pre-activations (bf16 or fp32).  Returns h or
    (h, c_last).  c_states, if given, is a [T,B,D] fp32 tensor that receives
    every cell state (the input sru_bwd needs)."""
    lib = load()
    if z_f.dim() != 3:
        raise ValueError("z_f must be [T,B,D]")
    T, B, D = (int(x) for x in z_f.shape)
    io = z_f.dtype
    for name, t in (("z_f", z_f), ("z_r", z_r), ("z_x", z_x)):
        _check_dev(name, t, io, z_f.shape)
    _check_dev("bias_f", bias_f, torch.float32, (D,))
    _check_dev("bias_r", bias_r, torch.float32, (D,))
    _check_dev("c0", c0, torch.float32, (B, D))
    _check_dev("c_states", c_states, torch.float32, z_f.shape)
    h = torch.empty_like(z_f) if out is None else out
    _check_dev("out", h, io, z_f.shape)
    c_last = torch.empty((B, D), dtype=torch.float32, device=z_f.device) if want_c_last else None
    nbytes = lib.lrs_sru_workspace_bytes(T, B, D)
    ws = _workspace(nbytes, z_f.device, workspace)
    _call(lib.lrs_sru_fwd_ex(_ptr(z_f), _ptr(z_r), _ptr(z_x), _ptr(bias_f), _ptr(bias_r), _ptr(c0),
                          _ptr(h), _ptr(c_last), _ptr(c_states), T, B, D, DTYPES[io], _ptr(ws),
                          nbytes, _stream(z_f.device), _opts(options)), "lrs_sru_fwd")
    return (h, c_last) if want_c_last else h


def sru_bwd(z_f, z_r, z_x, bias_f, bias_r, c_states, grad_h, c0=None, grad_c_last=None,
            out=None, workspace=None):
    """Backward of sru_fwd.  c_states: the [T,B,D] fp32 cell states sru_fwd
    saved; grad_h: dL/dh in the I/O type; grad_c_last: dL/dc_T [B,D] or None.
    Returns (grad_zf, grad_zr, grad_zx, grad_bias_f, grad_bias_r, grad_c0)."""
    lib = load()
    T, B, D = (int(x) for x in z_f.shape)
    io = z_f.dtype
    for name, t in (("z_f", z_f), ("z_r", z_r), ("z_x", z_x), ("grad_h", grad_h)):
        _check_dev(name, t, io, z_f.shape)
    _check_dev("bias_f", bias_f, torch.float32, (D,))
    _check_dev("bias_r", bias_r, torch.float32, (D,))
    _check_dev("c_states", c_states, torch.float32, z_f.shape)
    _check_dev("c0", c0, torch.float32, (B, D))
    _check_dev("grad_c_last", grad_c_last, torch.float32, (B, D))
    dev = z_f.device
    if out is None:
        out = (torch.empty_like(z_f), torch.empty_like(z_f), torch.empty_like(z_f),
               torch.empty(D, dtype=torch.float32, device=dev),
               torch.empty(D, dtype=torch.float32, device=dev),
               torch.empty((B, D), dtype=torch.float32, device=dev))
    dzf, dzr, dzx, dbf, dbr, dc0 = out
    nbytes = lib.lrs_sru_bwd_workspace_bytes(T, B, D)
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.lrs_sru_bwd(_ptr(z_f), _ptr(z_r), _ptr(z_x), _ptr(bias_f), _ptr(bias_r), _ptr(c0),
                          _ptr(c_states), _ptr(grad_h), _ptr(grad_c_last), _ptr(dzf), _ptr(dzr),
                          _ptr(dzx), _ptr(dbf), _ptr(dbr), _ptr(dc0), T, B, D, DTYPES[io],
                          _ptr(ws), nbytes, _stream(dev)), "lrs_sru_bwd")
    return dzf, dzr, dzx, dbf, dbr, dc0


def sru_deer_fwd(z_f, z_r, z_x, bias_f, bias_r, v_f, c0=None, c_init=None, eps: float = 1e-5,
                 k_max: int = 5, want_c_last: bool = False, out=None, c_states=None,
                 workspace=None, sync: bool = True, options=None):
    """SRU layer with v_f * c_{t-1} in the forget gate, by DEER.  sync=True:
    returns (h, c_states, c_last or None, info), info = {"iters", "deltas",
    "converged", "status"} as for deer_solve.  sync=False: returns
    (h, c_states, c_last, workspace); deer_stats(workspace, k_max) reads info."""
    lib = load()
    if z_f.dim() != 3:
        raise ValueError("z_f must be [T,B,D]")
    T, B, D = (int(x) for x in z_f.shape)
    io = z_f.dtype
    for name, t in (("z_f", z_f), ("z_r", z_r), ("z_x", z_x)):
        _check_dev(name, t, io, z_f.shape)
    for name, t in (("bias_f", bias_f), ("bias_r", bias_r), ("v_f", v_f)):
        _check_dev(name, t, torch.float32, (D,))
    _check_dev("c0", c0, torch.float32, (B, D))
    _check_dev("c_init", c_init, torch.float32, z_f.shape)
    h = torch.empty_like(z_f) if out is None else out
    _check_dev("out", h, io, z_f.shape)
    cs = torch.empty(z_f.shape, dtype=torch.float32, device=z_f.device) if c_states is None \
        else c_states
    _check_dev("c_states", cs, torch.float32, z_f.shape)
    c_last = torch.empty((B, D), dtype=torch.float32, device=z_f.device) if want_c_last else None
    nbytes = lib.lrs_sru_deer_workspace_bytes(T, B, D, int(k_max))
    ws = _workspace(nbytes, z_f.device, workspace)
    if sync:
        iters = ctypes.c_int(0)
        conv = ctypes.c_int(0)
        deltas = (ctypes.c_float * max(1, int(k_max)))()
        rc = lib.lrs_sru_deer_fwd_ex(_ptr(z_f), _ptr(z_r), _ptr(z_x), _ptr(bias_f), _ptr(bias_r),
                                  _ptr(v_f), _ptr(c0), _ptr(c_init), _ptr(h), _ptr(cs),
                                  _ptr(c_last), T, B, D, DTYPES[io], float(eps), int(k_max),
                                  ctypes.byref(iters), deltas, ctypes.byref(conv), _ptr(ws),
                                  nbytes, _stream(z_f.device), _opts(options))
        if rc not in (LRS_OK, LRS_ERR_NONFINITE):
            raise LrsError(rc, "lrs_sru_deer_fwd")
        info = {"iters": iters.value, "deltas": [float(deltas[i]) for i in range(iters.value)],
                "converged": bool(conv.value), "status": int(rc)}
        return h, cs, c_last, info
    _call(lib.lrs_sru_deer_fwd_ex(_ptr(z_f), _ptr(z_r), _ptr(z_x), _ptr(bias_f), _ptr(bias_r),
                               _ptr(v_f), _ptr(c0), _ptr(c_init), _ptr(h), _ptr(cs),
                               _ptr(c_last), T, B, D, DTYPES[io], float(eps), int(k_max), None,
                               None, None, _ptr(ws), nbytes, _stream(z_f.device), _opts(options)),
          "lrs_sru_deer_fwd")
    return h, cs, c_last, ws


def lstm_fwd(z_f, z_i, z_c, z_o, c0=None, want_c_last: bool = False, out=None, workspace=None,
             c_states=None, options=None):
    """LSTM cell-state layer with input-only gates on [T,B,D] pre-activations
    (bf16 or fp32).  Returns h or (h, c_last).  c_states, if given, is a
    [T,B,D] fp32 tensor that receives every cell state (lstm_bwd's input)."""
    lib = load()
    if z_f.dim() != 3:
        raise ValueError("z_f must be [T,B,D]")
    T, B, D = (int(x) for x in z_f.shape)
    io = z_f.dtype
    for name, t in (("z_f", z_f), ("z_i", z_i), ("z_c", z_c), ("z_o", z_o)):
        _check_dev(name, t, io, z_f.shape)
    _check_dev("c0", c0, torch.float32, (B, D))
    _check_dev("c_states", c_states, torch.float32, z_f.shape)
    h = torch.empty_like(z_f) if out is None else out
    _check_dev("out", h, io, z_f.shape)
    c_last = torch.empty((B, D), dtype=torch.float32, device=z_f.device) if want_c_last else None
    nbytes = lib.lrs_lstm_workspace_bytes(T, B, D)
    ws = _workspace(nbytes, z_f.device, workspace)
    _call(lib.lrs_lstm_fwd_ex(_ptr(z_f), _ptr(z_i), _ptr(z_c), _ptr(z_o), _ptr(c0), _ptr(h),
                              _ptr(c_last), _ptr(c_states), T, B, D, DTYPES[io], _ptr(ws), nbytes,
                              _stream(z_f.device), _opts(options)), "lrs_lstm_fwd")
    return (h, c_last) if want_c_last else h


def lstm_bwd(z_f, z_i, z_c, z_o, c_states, grad_h, c0=None, grad_c_last=None,
             want_grad_c0: bool = True, out=None, workspace=None):
    """Backward of lstm_fwd.  c_states: the [T,B,D] fp32 cell states lstm_fwd
    saved; grad_h: dL/dh in the I/O type; grad_c_last: dL/dc_T [B,D] or None.
    Returns (grad_zf, grad_zi, grad_zc, grad_zo, grad_c0 or None)."""
    lib = load()
    T, B, D = (int(x) for x in z_f.shape)
    io = z_f.dtype
    for name, t in (("z_f", z_f), ("z_i", z_i), ("z_c", z_c), ("z_o", z_o), ("grad_h", grad_h)):
        _check_dev(name, t, io, z_f.shape)
    _check_dev("c_states", c_states, torch.float32, z_f.shape)
    _check_dev("c0", c0, torch.float32, (B, D))
    _check_dev("grad_c_last", grad_c_last, torch.float32, (B, D))
    dev = z_f.device
    if out is None:
        out = (torch.empty_like(z_f), torch.empty_like(z_f), torch.empty_like(z_f),
               torch.empty_like(z_f),
               torch.empty((B, D), dtype=torch.float32, device=dev) if want_grad_c0 else None)
    dzf, dzi, dzc, dzo, dc0 = out
    for name, t in (("grad_zf", dzf), ("grad_zi", dzi), ("grad_zc", dzc), ("grad_zo", dzo)):
        _check_dev(name, t, io, z_f.shape)
    _check_dev("grad_c0", dc0, torch.float32, (B, D))
    nbytes = lib.lrs_lstm_workspace_bytes(T, B, D)
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.lrs_lstm_bwd(_ptr(z_f), _ptr(z_i), _ptr(z_c), _ptr(z_o), _ptr(c0), _ptr(c_states),
                           _ptr(grad_h), _ptr(grad_c_last), _ptr(dzf), _ptr(dzi), _ptr(dzc),
                           _ptr(dzo), _ptr(dc0), T, B, D, DTYPES[io], _ptr(ws), nbytes,
                           _stream(dev)), "lrs_lstm_bwd")
    return dzf, dzi, dzc, dzo, dc0


def deer_solve(w, u, h0=None, h_init=None, eps: float = 1e-5, k_max: int = 5, out=None,
               workspace=None, sync: bool = True, options=None):
    """DEER Newton solve of h_t = tanh(w h_{t-1} + u_t); u: [B,D,T] fp32, w: [D].

    sync=True: returns (h, info) with info = {"iters", "deltas", "converged",
    "status"}; a non-finite final update is reported in info["status"] rather
    than raised.  sync=False: enqueues the solve without waiting and returns
    (h, workspace); deer_stats(workspace, k_max) reads info later."""
    lib = load()
    B, D, T = _dims(u, "bdt")
    _check_dev("u", u, torch.float32, u.shape)
    _check_dev("w", w, torch.float32, (D,))
    _check_dev("h0", h0, torch.float32, (B, D))
    _check_dev("h_init", h_init, torch.float32, u.shape)
    h = torch.empty_like(u) if out is None else out
    _check_dev("out", h, torch.float32, u.shape)
    nbytes = lib.lrs_deer_workspace_bytes(B, D, T, k_max)
    ws = _workspace(nbytes, u.device, workspace)
    if not sync:
        rc = lib.lrs_deer_solve_ex(_ptr(w), _ptr(u), _ptr(h0), _ptr(h_init), _ptr(h), B, D, T,
                                float(eps), int(k_max), None, None, None, _ptr(ws), nbytes,
                                _stream(u.device), _opts(options))
        if rc != LRS_OK:
            raise LrsError(rc, "lrs_deer_solve")
        return h, ws
    iters = ctypes.c_int(0)
    conv = ctypes.c_int(0)
    deltas = (ctypes.c_float * max(k_max, 1))()
    rc = lib.lrs_deer_solve_ex(_ptr(w), _ptr(u), _ptr(h0), _ptr(h_init), _ptr(h), B, D, T,
                            float(eps), int(k_max), ctypes.byref(iters), deltas,
                            ctypes.byref(conv), _ptr(ws), nbytes, _stream(u.device), _opts(options))
    if rc not in (LRS_OK, LRS_ERR_NONFINITE):
        raise LrsError(rc, "lrs_deer_solve")
    info = {"iters": iters.value, "deltas": [float(deltas[i]) for i in range(iters.value)],
            "converged": bool(conv.value), "status": int(rc)}
    return h, info


def deer_solve_seq(w, u, h0=None, h_init=None, eps: float = 1e-5, k_max: int = 5, out=None,
                   workspace=None, sync: bool = True, options=None):
    """deer_solve with per-sequence stopping (each batch entry stops on its own
    norm).  Returns (h, iters[B], converged[B]) when sync, else (h, workspace)."""
    lib = load()
    B, D, T = (int(x) for x in u.shape)
    _check_dev("u", u, torch.float32, u.shape)
    _check_dev("w", w, torch.float32, (D,))
    _check_dev("h0", h0, torch.float32, (B, D))
    _check_dev("h_init", h_init, torch.float32, u.shape)
    h = torch.empty_like(u) if out is None else out
    _check_dev("out", h, torch.float32, u.shape)
    nbytes = lib.lrs_deer_seq_workspace_bytes(B, D, T, int(k_max))
    ws = _workspace(nbytes, u.device, workspace)
    if sync:
        iters = (ctypes.c_int * max(B, 1))()
        conv = (ctypes.c_int * max(B, 1))()
        rc = lib.lrs_deer_solve_seq_ex(_ptr(w), _ptr(u), _ptr(h0), _ptr(h_init), _ptr(h), B, D, T,
                                    float(eps), int(k_max), iters, conv, _ptr(ws), nbytes,
                                    _stream(u.device), _opts(options))
        if rc not in (LRS_OK, LRS_ERR_NONFINITE):  # non-finite updates show as not converged
            raise LrsError(rc, "lrs_deer_solve_seq")
        return h, [int(iters[b]) for b in range(B)], [bool(conv[b]) for b in range(B)]
    _call(lib.lrs_deer_solve_seq_ex(_ptr(w), _ptr(u), _ptr(h0), _ptr(h_init), _ptr(h), B, D, T,
                                 float(eps), int(k_max), None, None, _ptr(ws), nbytes,
                                 _stream(u.device), _opts(options)), "lrs_deer_solve_seq")
    return h, ws


def deer_eps_schedule(step: int, total_steps: int, early: float = 1e-4, late: float = 1e-6) -> float:
    """Newton tolerance for training step `step` of `total_steps`
    (lrs_deer_eps_schedule: log-linear from `early` to `late`)."""
    return float(load().lrs_deer_eps_schedule(int(step), int(total_steps), float(early),
                                              float(late)))


def deer_bwd(w, h, grad_h, h0=None, want_grad_h0: bool = True, out=None, workspace=None):
    """Backward of h_t = tanh(w h_{t-1} + u_t) at the solution h [B,D,T] (e.g.
    deer_solve's result) for dL/dh = grad_h.  Returns (grad_u, grad_w, grad_h0)."""
    lib = load()
    B, D, T = _dims(h, "bdt")
    _check_dev("h", h, torch.float32, h.shape)
    _check_dev("grad_h", grad_h, torch.float32, h.shape)
    _check_dev("w", w, torch.float32, (D,))
    _check_dev("h0", h0, torch.float32, (B, D))
    dev = h.device
    if out is None:
        out = (torch.empty_like(h), torch.empty(D, dtype=torch.float32, device=dev),
               torch.empty((B, D), dtype=torch.float32, device=dev) if want_grad_h0 else None)
    gu, gw, gh0 = out
    nbytes = lib.lrs_deer_bwd_workspace_bytes(B, D, T)
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.lrs_deer_bwd(_ptr(w), _ptr(h0), _ptr(h), _ptr(grad_h), _ptr(gu), _ptr(gw), _ptr(gh0),
                           B, D, T, _ptr(ws), nbytes, _stream(dev)), "lrs_deer_bwd")
    return gu, gw, gh0


def rnn_seq(w, u, h0=None, out=None):
    """h_t = tanh(w h_{t-1} + u_t) over u [B,D,T] fp32, evaluated step after
    step with one lane per channel (lrs_rnn_seq); the sequential reference for
    deer_solve.  Returns h [B,D,T]."""
    lib = load()
    B, D, T = _dims(u, "bdt")
    _check_dev("u", u, torch.float32, u.shape)
    _check_dev("w", w, torch.float32, (D,))
    _check_dev("h0", h0, torch.float32, (B, D))
    h = torch.empty_like(u) if out is None else out
    _check_dev("out", h, torch.float32, u.shape)
    _call(lib.lrs_rnn_seq(_ptr(w), _ptr(u), _ptr(h0), _ptr(h), B, D, T, _stream(u.device)),
          "lrs_rnn_seq")
    return h


def deer_stats(workspace, k_max: int = 5):
    """Record of the last solve run with `workspace` (see deer_solve): waits for
    the current stream and returns {"iters", "deltas", "converged", "status"}."""
    lib = load()
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise TypeError("workspace must be the device tensor a solve used")
    iters = ctypes.c_int(0)
    conv = ctypes.c_int(0)
    deltas = (ctypes.c_float * max(k_max, 1))()
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib.lrs_deer_stats(_ptr(workspace), nbytes, int(k_max), ctypes.byref(iters), deltas,
                            ctypes.byref(conv), _stream(workspace.device))
    if rc not in (LRS_OK, LRS_ERR_NONFINITE):
        raise LrsError(rc, "lrs_deer_stats")
    return {"iters": iters.value, "deltas": [float(deltas[i]) for i in range(iters.value)],
            "converged": bool(conv.value), "status": int(rc)}
