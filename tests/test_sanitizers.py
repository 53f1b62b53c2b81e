"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (oracle/lrs_oracle.c) is rebuilt with gcc's ASan + UBSan
  (no recovery: the first report aborts), every one of its functions runs on
  small inputs of awkward shapes (T = 1, one channel, ragged sizes, optional
  arguments present and absent) in a child process that preloads the ASan
  runtime, and the outputs must equal the regular build's bit for bit (same
  optimisation and floating-point flags).
* The HIP library's host code (argument validation, workspace queries, launch
  planning) is rebuilt with clang's ASan + UBSan on the host side only
  (-Xarch_host before each -fsanitize=; the device code is unchanged) and the
  ABI tests run against it in a child process that preloads clang's ASan
  runtime.  Those tests make no HIP runtime call, so no GPU is needed.
"""
import glob
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "lrs_oracle.c")
CSRC = os.path.join(ROOT, "linear_recurrence_scan_diagonal_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

# Every oracle function on small inputs; results saved for comparison.
BATTERY = r'''
import sys, numpy as np
sys.path.insert(0, ROOT)
import oracle
oracle._LIB_PATH = LIB
rng = np.random.default_rng(5)
out = {}
def put(tag, res):
    if isinstance(res, dict):
        for k, v in res.items(): out[f"{tag}/{k}"] = np.asarray(v, dtype=np.float64)
    elif isinstance(res, tuple):
        for i, v in enumerate(res): out[f"{tag}/{i}"] = np.asarray(v, dtype=np.float64)
    else:
        out[tag] = np.asarray(res, dtype=np.float64)
for (C, T) in [(1, 1), (3, 17), (2, 64)]:
    a = rng.uniform(0.5, 1.0, (C, T)); b = rng.normal(size=(C, T)); g = rng.normal(size=(C, T))
    h0 = rng.normal(size=C)
    for useh0 in (False, True):
        x0 = h0 if useh0 else None
        h = oracle.scan_fwd(a, b, x0)
        put(f"scan_fwd/{C}/{T}/{useh0}", h)
        put(f"scan_bwd/{C}/{T}/{useh0}", oracle.scan_bwd(a, h, x0, g))
for (T, B, D) in [(1, 1, 1), (5, 2, 3), (33, 1, 4)]:
    z = [rng.normal(size=(T, B, D)) for _ in range(5)]
    bf, br, vf = rng.normal(-1, 0.1, D), rng.normal(-1, 0.1, D), rng.uniform(-0.25, 0.25, D)
    c0 = rng.normal(size=(B, D)); gcl = rng.normal(size=(B, D))
    for usec0 in (False, True):
        c = c0 if usec0 else None
        tag = f"{T}/{B}/{D}/{usec0}"
        put("sru_fwd/" + tag, oracle.sru_fwd(z[0], z[1], z[2], bf, br, c))
        put("sru_bwd/" + tag, oracle.sru_bwd(z[0], z[1], z[2], bf, br, z[3], c0=c,
                                             gcl=gcl if usec0 else None))
        put("lstm_fwd/" + tag, oracle.lstm_fwd(z[0], z[1], z[2], z[3], c))
        put("lstm_bwd/" + tag, oracle.lstm_bwd(z[0], z[1], z[2], z[3], z[4], c0=c,
                                               gcl=gcl if usec0 else None))
        put("sru_nl_seq/" + tag, oracle.sru_nl_seq(z[0], z[1], z[2], bf, br, vf, c))
        r = oracle.sru_deer(z[0], z[1], z[2], bf, br, vf, c, k_max=4)
        put("sru_deer/" + tag, (r[0], r[1], r[2], r[3]))
for (B, D, T) in [(1, 1, 1), (2, 3, 19)]:
    w = rng.uniform(-0.9, 0.9, D); u = rng.normal(size=(B, D, T)); h0 = rng.normal(size=(B, D))
    g = rng.normal(size=(B, D, T))
    for useh0 in (False, True):
        x0 = h0 if useh0 else None
        tag = f"{B}/{D}/{T}/{useh0}"
        put("rnn_seq/" + tag, oracle.rnn_seq(w, u, x0))
        hd, it, dl = oracle.deer(w, u, x0, k_max=6)
        put("deer/" + tag, (hd, it, dl))
        put("deer_bwd/" + tag, oracle.deer_bwd(w, hd, g, x0))
np.savez(OUT, **out)
print("battery done", len(out))
'''


def _clean(res):
    bad = [s for s in ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehavior")
           if s in res.stderr]
    return res.returncode == 0 and not bad


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc's ASan runtime not available")
    common = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]
    libs = {}
    for kind, extra in (("plain", []), ("san", ["-g", "-fsanitize=address,undefined",
                                                "-fno-sanitize-recover=all",
                                                "-fno-omit-frame-pointer"])):
        libs[kind] = str(tmp_path / f"liblrs_oracle_{kind}.so")
        subprocess.run(["gcc", *common, *extra, "-o", libs[kind], ORACLE_SRC, "-lm"], check=True)
    outs = {}
    for kind in ("plain", "san"):
        out = str(tmp_path / f"out_{kind}.npz")
        script = f"ROOT = {ROOT!r}\nLIB = {libs[kind]!r}\nOUT = {out!r}\n" + BATTERY
        env = dict(os.environ, OMP_NUM_THREADS="2")
        if kind == "san":
            env.update(LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
        res = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                             env=env, timeout=300)
        assert _clean(res), f"{kind} oracle battery failed:\n{res.stdout}\n{res.stderr[-4000:]}"
        outs[kind] = dict(np.load(out))
    assert outs["plain"].keys() == outs["san"].keys() and len(outs["plain"]) > 100
    for k, v in outs["plain"].items():
        assert np.array_equal(v, outs["san"][k]), k


def test_library_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    rt = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                       "libclang_rt.asan-x86_64.so")))
    if not rt:
        pytest.skip("clang's ASan runtime not available")
    flags = [f"--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"),
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    procs, objs = [], []
    for src in sources:
        obj = str(tmp_path / (src[:-4] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE))
    for p, src in zip(procs, sources):
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{src}: {err.decode()[-2000:]}"
    lib = str(tmp_path / "liblrs_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs],
                   check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               LRS_TEST_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True,
                         text=True, env=env, cwd=ROOT, timeout=600)
    assert _clean(res) and " passed" in res.stdout, \
        f"ABI tests under sanitizers failed:\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
