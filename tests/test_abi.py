"""The C-ABI library loads without a GPU, exports every function include/lrs.h
declares, and its host-side validation and workspace queries behave as the
header states.  No call here reaches a HIP runtime function."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrs.h")
# LRS_TEST_LIB: run these tests against another build of the same sources
# (the sanitizer test uses it for a host-instrumented copy)
LIB = os.environ.get("LRS_TEST_LIB") or os.path.join(ROOT, "linear_recurrence_scan_diagonal_amd",
                                                     "liblrs.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="liblrs.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LRS_API\s+[\w\s\*]*?\b(lrs_\w+)\s*\(", text)))


def header_constants():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(LRS_\w+)\s+(\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    from linear_recurrence_scan_diagonal_amd import binding
    if binding._lib is None:
        binding.LIB_PATH = LIB
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 34, names
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in lrs.h but not exported"


def test_binding_covers_exports():
    from linear_recurrence_scan_diagonal_amd import binding
    assert sorted(binding.EXPORTS) == declared_functions()


def test_constants_match_binding():
    from linear_recurrence_scan_diagonal_amd import binding
    c = header_constants()
    assert c["LRS_OK"] == binding.LRS_OK and c["LRS_ERR_NONFINITE"] == binding.LRS_ERR_NONFINITE
    assert c["LRS_ERR_WORKSPACE"] == binding.LRS_ERR_WORKSPACE
    assert c["LRS_LAYOUT_BDT"] == binding.LAYOUTS["bdt"] and c["LRS_LAYOUT_TBD"] == binding.LAYOUTS["tbd"]
    assert c["LRS_F32"] == 0 and c["LRS_BF16"] == 1


def test_status_strings(lib):
    for code in range(6):
        assert lib.lrs_status_string(code).startswith(b"LRS_")
    assert lib.lrs_status_string(99) == b"LRS_ERR_UNKNOWN"
    assert lib.lrs_version() >= 100


def test_scan_workspace_queries(lib):
    # a channel that fits one workgroup needs no look-back workspace
    assert lib.lrs_scan_workspace_bytes(8, 512, 4096, 0, 0) == 0
    # a million-step channel does: one 8-byte word per chunk plus one ticket
    # per channel, with chunks of at most 16384 steps
    big = lib.lrs_scan_workspace_bytes(2, 256, 1 << 20, 0, 0)
    assert big >= 512 * 64 * 8 + 512 * 4
    assert lib.lrs_scan_workspace_bytes(-1, 1, 1, 0, 0) == 0
    assert lib.lrs_scan_workspace_bytes(1, 1, 1, 7, 0) == 0
    assert lib.lrs_scan_workspace_bytes(1 << 40, 1 << 40, 2, 0, 0) == 0  # overflow
    assert lib.lrs_deer_workspace_bytes(16, 512, 8192, 5) >= 16 * 512 * 8192 * 4
    assert lib.lrs_deer_workspace_bytes(1, 1, 1, 0) == 0
    # SRU backward: per-tile bias partials (2 floats per channel and time block)
    assert lib.lrs_sru_bwd_workspace_bytes(2048, 32, 1024) >= 2 * 32 * 32768 * 4
    assert lib.lrs_sru_bwd_workspace_bytes(-1, 1, 1) == 0
    # DEER backward: one dL/dw partial per channel and chunk
    assert lib.lrs_deer_bwd_workspace_bytes(16, 512, 8192) >= 16 * 512 * 4
    assert lib.lrs_deer_bwd_workspace_bytes(1, 1, -3) == 0
    # LSTM: look-back words once a channel spans several time blocks
    assert lib.lrs_lstm_workspace_bytes(2048, 32, 1024) >= 32 * 1024 * (2048 // 64) * 8
    assert lib.lrs_lstm_workspace_bytes(16, 4, 8) == 0
    assert lib.lrs_lstm_workspace_bytes(-1, 1, 1) == 0


def test_validation_before_any_launch(lib):
    from linear_recurrence_scan_diagonal_amd import binding as b
    p = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    null = None
    # negative size, bad layout, bad dtype, null pointers, misalignment
    assert lib.lrs_scan_fwd(p, p, null, p, -1, 1, 1, 0, 0, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_scan_fwd(p, p, null, p, 1, 1, 1, 5, 0, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_scan_fwd(p, p, null, p, 1, 1, 1, 0, 9, null, 0, null) == b.LRS_ERR_INVALID_ARG
    # bf16 arrays: 2-byte alignment, and extents of 2 bytes per element (h six
    # bytes past a overlaps a's four elements)
    assert lib.lrs_scan_fwd(ctypes.c_void_p(0x1001), ctypes.c_void_p(0x2000), null,
                            ctypes.c_void_p(0x9000), 1, 1, 4, 0, 1, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_scan_fwd(p, ctypes.c_void_p(0x2000), null, ctypes.c_void_p(0x1006), 1, 1, 4, 0, 1,
                            null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_scan_fwd(null, p, null, p, 1, 1, 4, 0, 0, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_scan_fwd(ctypes.c_void_p(0x1002), p, null, ctypes.c_void_p(0x9000), 1, 1, 4, 0, 0,
                            null, 0, null) == b.LRS_ERR_INVALID_ARG
    # output overlapping an input
    assert lib.lrs_scan_fwd(p, ctypes.c_void_p(0x8000), null, ctypes.c_void_p(0x1008), 1, 1, 64, 0,
                            0, null, 0, null) == b.LRS_ERR_INVALID_ARG
    # a multi-chunk channel without workspace
    assert lib.lrs_scan_fwd(ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000000), null,
                            ctypes.c_void_p(0x400000000), 1, 1, 1 << 20, 0, 0, null, 0,
                            null) == b.LRS_ERR_WORKSPACE
    # empty problems are valid and do nothing
    assert lib.lrs_scan_fwd(null, null, null, null, 0, 5, 7, 0, 0, null, 0, null) == b.LRS_OK
    assert lib.lrs_scan_fwd(null, null, null, null, 3, 5, 0, 1, 0, null, 0, null) == b.LRS_OK
    # backward: grad_a aliasing a is rejected, grad_b == grad_h is accepted past the alias check
    q = ctypes.c_void_p
    assert lib.lrs_scan_bwd(q(0x10000), q(0x20000), null, q(0x30000), q(0x10000), q(0x40000), null,
                            1, 1, 64, 0, 0, null, 0, null) == b.LRS_ERR_INVALID_ARG
    # sequential RNN: null u, negative size, misaligned h, h overlapping u; empty is valid
    assert lib.lrs_rnn_seq(p, null, null, q(0x9000), 1, 1, 4, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_rnn_seq(p, p, null, q(0x9000), 1, -1, 4, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_rnn_seq(q(0x100), q(0x1000), null, q(0x9002), 1, 1, 4, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_rnn_seq(q(0x100), q(0x1000), null, q(0x1008), 1, 1, 4, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_rnn_seq(null, null, null, null, 2, 3, 0, null) == b.LRS_OK
    # SRU and DEER argument checks
    assert lib.lrs_sru_fwd(p, p, p, p, p, null, p, null, null, 4, 1, 1, 3, null, 0,
                           null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_fwd(null, p, p, p, p, null, p, null, null, 4, 1, 1, 1, null, 0,
                           null) == b.LRS_ERR_INVALID_ARG
    # the saved cell states must not overlap an input
    assert lib.lrs_sru_fwd(q(0x10000), q(0x20000), q(0x30000), q(0x40000), q(0x50000), null,
                           q(0x60000), null, q(0x10000), 4, 1, 1, 1, null, 0,
                           null) == b.LRS_ERR_INVALID_ARG
    # SRU backward: missing saved states, bad dtype, an output overlapping an input
    assert lib.lrs_sru_bwd(p, p, p, p, p, null, null, p, null, p, p, p, p, p, null, 4, 1, 1, 1,
                           null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_bwd(p, p, p, p, p, null, p, p, null, p, p, p, p, p, null, 4, 1, 1, 7,
                           null, 0, null) == b.LRS_ERR_INVALID_ARG
    zs = [q(0x10000 * (i + 1)) for i in range(12)]
    assert lib.lrs_sru_bwd(zs[0], zs[1], zs[2], zs[3], zs[4], null, zs[5], zs[6], null,
                           zs[0], zs[7], zs[8], zs[9], zs[10], null, 4, 1, 1, 1, null, 0,
                           null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_bwd(zs[0], zs[1], zs[2], zs[3], zs[4], null, zs[5], zs[6], null,
                           zs[11], zs[7], zs[8], zs[9], zs[10], null, 4, 1, 1, 1, null, 0,
                           null) == b.LRS_ERR_WORKSPACE
    assert lib.lrs_deer_solve(p, p, null, null, p, 1, 1, 4, ctypes.c_float(1e-5), 0, None, None, None,
                              null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_deer_solve(q(0x10000), q(0x20000), null, null, q(0x90000), 1, 1, 4,
                              ctypes.c_float(1e-5), 5, None, None, None, null, 0,
                              null) == b.LRS_ERR_WORKSPACE
    assert lib.lrs_deer_stats(null, 0, 5, None, None, None, null) == b.LRS_ERR_WORKSPACE
    # DEER backward: missing h, an output overlapping an input, missing workspace
    assert lib.lrs_deer_bwd(p, null, null, p, p, p, null, 1, 1, 4, null, 0,
                            null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_deer_bwd(q(0x10000), null, q(0x20000), q(0x30000), q(0x20000), q(0x40000), null,
                            1, 1, 4, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_deer_bwd(q(0x10000), null, q(0x20000), q(0x30000), q(0x50000), q(0x40000), null,
                            1, 1, 4, null, 0, null) == b.LRS_ERR_WORKSPACE
    # LSTM forward: bad dtype, missing gate, saved states overlapping an input,
    # a multi-block time axis without workspace
    assert lib.lrs_lstm_fwd(p, p, p, p, null, p, null, null, 4, 1, 1, 2, null, 0,
                            null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_lstm_fwd(p, null, p, p, null, p, null, null, 4, 1, 1, 1, null, 0,
                            null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_lstm_fwd(zs[0], zs[1], zs[2], zs[3], null, zs[4], null, zs[2], 4, 1, 1, 1,
                            null, 0, null) == b.LRS_ERR_INVALID_ARG
    big = [q(0x1000000 * (i + 1)) for i in range(12)]
    assert lib.lrs_lstm_fwd(big[0], big[1], big[2], big[3], null, big[4], null, null, 1024, 1, 1,
                            1, null, 0, null) == b.LRS_ERR_WORKSPACE
    # LSTM backward: missing saved states, a gradient overlapping another,
    # a multi-block time axis without workspace
    assert lib.lrs_lstm_bwd(p, p, p, p, null, null, p, null, p, p, p, p, null, 4, 1, 1, 1, null,
                            0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_lstm_bwd(big[0], big[1], big[2], big[3], null, big[4], big[5], null, big[6],
                            big[7], big[7], big[8], null, 4, 1, 1, 1, null, 0,
                            null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_lstm_bwd(big[0], big[1], big[2], big[3], null, big[4], big[5], null, big[6],
                            big[7], big[8], big[9], null, 1024, 1, 1, 1, null, 0,
                            null) == b.LRS_ERR_WORKSPACE
    # fused forward + backward: h may be left out only where one kernel does
    # both passes ([B,D,T], T <= 8192); an output overlapping an input
    assert lib.lrs_scan_fwd_bwd(big[0], big[1], null, big[2], null, big[3], big[4], null, 1, 1,
                                16384, 0, 0, null, 0, null) == b.LRS_ERR_UNSUPPORTED
    assert lib.lrs_scan_fwd_bwd(big[0], big[1], null, big[2], null, big[3], big[4], null, 1, 1,
                                64, 1, 0, null, 0, null) == b.LRS_ERR_UNSUPPORTED
    assert lib.lrs_scan_fwd_bwd(big[0], big[1], null, big[2], big[1], big[3], big[4], null, 1, 1,
                                64, 0, 0, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_scan_fwd_bwd(big[0], big[1], null, big[2], big[5], big[3], big[4], null, 1, 1,
                                1 << 20, 0, 0, null, 0, null) == b.LRS_ERR_WORKSPACE
    # SRU by DEER: missing v_f or c_states, bad dtype, k_max 0, saved states
    # overlapping an input, missing workspace
    cf = ctypes.c_float(1e-5)
    assert lib.lrs_sru_deer_fwd(p, p, p, p, p, null, null, null, p, p, null, 4, 1, 1, 1, cf, 5,
                                None, None, None, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_deer_fwd(p, p, p, p, p, p, null, null, p, null, null, 4, 1, 1, 1, cf, 5,
                                None, None, None, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_deer_fwd(p, p, p, p, p, p, null, null, p, p, null, 4, 1, 1, 3, cf, 5,
                                None, None, None, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_deer_fwd(p, p, p, p, p, p, null, null, p, p, null, 4, 1, 1, 1, cf, 0,
                                None, None, None, null, 0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_deer_fwd(big[0], big[1], big[2], big[3], big[4], big[5], null, null,
                                big[6], big[0], null, 4, 1, 1, 1, cf, 5, None, None, None, null,
                                0, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_sru_deer_fwd(big[0], big[1], big[2], big[3], big[4], big[5], null, null,
                                big[6], big[7], null, 4, 1, 1, 1, cf, 5, None, None, None, null,
                                0, null) == b.LRS_ERR_WORKSPACE
    assert lib.lrs_sru_deer_workspace_bytes(2048, 32, 1024, 5) >= 32 * 1024 * 2048 * 4
    # DEER with per-sequence stopping: too many sequences, missing u, missing workspace
    assert lib.lrs_deer_solve_seq(p, p, null, null, p, 70000, 1, 1, cf, 5, None, None, null, 0,
                                  null) == b.LRS_ERR_UNSUPPORTED
    assert lib.lrs_deer_solve_seq(p, null, null, null, p, 2, 1, 4, cf, 5, None, None, null, 0,
                                  null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_deer_solve_seq(big[0], big[1], null, null, big[2], 2, 1, 4, cf, 5, None, None,
                                  null, 0, null) == b.LRS_ERR_WORKSPACE
    assert lib.lrs_deer_seq_workspace_bytes(16, 512, 8192, 5) >= 16 * 512 * 8192 * 4
    assert lib.lrs_deer_stats(p, 1 << 20, 0, None, None, None, null) == b.LRS_ERR_INVALID_ARG
    assert lib.lrs_deer_stats(p, 64, 5, None, None, None, null) == b.LRS_ERR_WORKSPACE


def test_product_path_has_no_fallback():
    """The package never imports the oracle, and the binding raises when the
    library is absent instead of computing anything itself."""
    pkg = os.path.join(ROOT, "linear_recurrence_scan_diagonal_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn
    from linear_recurrence_scan_diagonal_amd import binding
    saved, saved_lib = binding.LIB_PATH, binding._lib
    try:
        binding.LIB_PATH, binding._lib = "/nonexistent/liblrs.so", None
        with pytest.raises(RuntimeError):
            binding.load()
    finally:
        binding.LIB_PATH, binding._lib = saved, saved_lib


def test_deer_eps_schedule():
    """Log-linear from the loose to the tight tolerance over training, computed
    by the library (lrs_deer_eps_schedule), clamped outside the run, NaN for
    tolerances that are not positive and finite."""
    import math
    from linear_recurrence_scan_diagonal_amd import binding as b
    assert b.deer_eps_schedule(0, 101) == pytest.approx(1e-4, rel=1e-6)
    assert b.deer_eps_schedule(100, 101) == pytest.approx(1e-6, rel=1e-6)
    assert b.deer_eps_schedule(50, 101) == pytest.approx(1e-5, rel=1e-6)
    vals = [b.deer_eps_schedule(i, 11) for i in range(11)]
    assert all(x > y for x, y in zip(vals, vals[1:]))
    # each step multiplies by the same factor (late/early)^(1/10)
    ratios = [y / x for x, y in zip(vals, vals[1:])]
    assert all(r == pytest.approx(0.01 ** 0.1, rel=1e-6) for r in ratios)
    assert b.deer_eps_schedule(5, 1) == pytest.approx(1e-6, rel=1e-6)
    assert b.deer_eps_schedule(500, 101) == pytest.approx(1e-6, rel=1e-6)
    assert b.deer_eps_schedule(-3, 101) == pytest.approx(1e-4, rel=1e-6)
    assert b.deer_eps_schedule(3, 7, early=2e-3, late=2e-3) == pytest.approx(2e-3, rel=1e-6)
    assert math.isnan(b.deer_eps_schedule(3, 7, early=0.0, late=1e-6))
    assert math.isnan(b.deer_eps_schedule(3, 7, early=1e-4, late=-1.0))
    assert math.isnan(b.deer_eps_schedule(3, 7, early=float("inf"), late=1e-6))


def test_options_struct_and_ex_validation(lib):
    """lrs_options_default sets every field to -1 (reserved 0); the _ex entry
    points validate exactly as the plain ones, with or without options."""
    from linear_recurrence_scan_diagonal_amd import binding as b
    assert ctypes.sizeof(b.LrsOptions) == 40
    o = b.LrsOptions()
    o.reserved = 99
    lib.lrs_options_default(ctypes.byref(o))
    assert (o.serial_fwd_max_t, o.serial_bwd_max_t, o.packed_max_t, o.persist_min_blocks,
            o.deer_fuse, o.reserved) == (-1, -1, -1, -1, -1, 0)
    lib.lrs_options_default(None)  # a no-op
    null = None
    p = ctypes.c_void_p(1 << 20)
    for opt in (None, ctypes.byref(o)):
        assert lib.lrs_scan_fwd_ex(null, p, null, p, 1, 1, 8, 0, 0, null, 0, null,
                                   opt) == b.LRS_ERR_INVALID_ARG
        assert lib.lrs_scan_bwd_ex(p, p, null, p, p, p, null, 1, 1, -8, 0, 0, null, 0, null,
                                   opt) == b.LRS_ERR_INVALID_ARG
        assert lib.lrs_scan_fwd_bwd_ex(p, p, null, p, p, p, p, null, 1, 1, 8, 5, 0, null, 0, null,
                                       opt) == b.LRS_ERR_INVALID_ARG
        assert lib.lrs_sru_fwd_ex(p, null, p, p, p, null, p, null, null, 4, 1, 8, 1, null, 0,
                                  null, opt) == b.LRS_ERR_INVALID_ARG
        assert lib.lrs_deer_solve_ex(p, p, null, null, p, 1, 1, 8, ctypes.c_float(1e-5), 0, None,
                                     None, None, null, 0, null, opt) == b.LRS_ERR_INVALID_ARG
        assert lib.lrs_deer_solve_seq_ex(p, null, null, null, p, 2, 1, 4, ctypes.c_float(1e-5), 5,
                                         None, None, null, 0, null, opt) == b.LRS_ERR_INVALID_ARG
        assert lib.lrs_sru_deer_fwd_ex(p, p, p, p, p, p, null, null, p, p, null, 4, 1, 8, 9,
                                       ctypes.c_float(1e-5), 5, None, None, None, null, 0, null,
                                       opt) == b.LRS_ERR_INVALID_ARG
