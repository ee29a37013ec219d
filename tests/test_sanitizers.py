"""AddressSanitizer and UndefinedBehaviorSanitizer over the CPU-side code.

Two legs, each in a process of its own (gcc's and clang's sanitizer runtimes
cannot share one):
  - the oracle, rebuilt with gcc -fsanitize=address,undefined, driven through
    every entry point (forward and backward with and without S_in / dS_out,
    empty and one-token chunks, chained chunks, the short convolution);
  - the C-ABI host layer (sf_gdn_api.cpp: argument checks, plans, workspace
    sizes, error strings, profiler), rebuilt with the sanitizers on its host
    code only and linked with the already built kernel objects, under the
    host tests of test_host.py (no GPU call: every case there fails or plans
    before a launch).
A report stops the process (halt_on_error) and fails the test.
"""
import os
import subprocess
import sys
import tempfile

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(REPO, "linear_recurrence_chunked_gated_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

_ORACLE_DRIVER = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle.gdn as og
og._LIB = sys.argv[2]
lib = og._load()
assert lib._name == sys.argv[2], lib._name
rng = np.random.default_rng(5)

def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)

n = 0
for B, T, H, D in [(1, 0, 2, 8), (1, 1, 1, 8), (2, 67, 3, 16), (1, 130, 2, 64)]:
    q, k = unit(rng.normal(size=(B, T, H, D))), unit(rng.normal(size=(B, T, H, D)))
    v = rng.normal(size=(B, T, H, D))
    a = np.exp(-np.log1p(np.exp(rng.normal(size=(B, T, H)))))
    b = 1 / (1 + np.exp(-rng.normal(size=(B, T, H))))
    S = rng.normal(scale=0.1, size=(B, H, D, D))
    dS = rng.normal(scale=0.1, size=(B, H, D, D))
    for s_in in (None, S):
        o, _ = og.gdn_fwd(q, k, v, a, b, s_in)
        dO = rng.normal(size=o.shape)
        for ds in (None, dS):
            og.gdn_bwd(q, k, v, a, b, s_in, dO, ds)
            n += 1
    if T >= 3:
        L = [T // 3, T // 3, T - 2 * (T // 3)]
        og.gdn_fwd_chained(q, k, v, a, b, S, L)
        og.gdn_bwd_chained(q, k, v, a, b, S, rng.normal(size=v.shape), dS, L)
        n += 1
for B, T, C, W in [(1, 0, 4, 4), (2, 37, 16, 4), (1, 5, 8, 2)]:
    x, w = rng.normal(size=(B, T, C)), rng.normal(size=(C, W))
    cin = rng.normal(size=(B, W - 1, C))
    for act in (0, 1):
        for c in (None, cin):
            y, cout = og.shortconv_fwd(x, w, c, act)
            og.shortconv_bwd(x, w, c, rng.normal(size=y.shape), rng.normal(size=cout.shape), act)
            n += 1
print("oracle calls", n)
"""

_HOST_DRIVER = r"""
import os, sys
repo, lib = sys.argv[1], sys.argv[2]
sys.path.insert(0, repo)
sys.path.insert(0, os.path.join(repo, "tests"))
import pytest
from linear_recurrence_chunked_gated_amd import _lib
_lib.LIB_PATH = lib
assert _lib.load()._name == lib
sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                      os.path.join(repo, "tests", "test_host.py")]))
"""


def _run(driver, lib, preload, tmp):
    path = os.path.join(tmp, "driver.py")
    with open(path, "w") as f:
        f.write(driver)
    env = dict(os.environ, LD_PRELOAD=preload, **ENV)
    r = subprocess.run([sys.executable, path, REPO, lib], env=env, capture_output=True,
                       text=True, timeout=600, cwd=tmp)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's libasan is not installed")
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "libgdn_oracle.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-o", lib,
                        os.path.join(REPO, "oracle", "gdn_oracle.c"), "-lm"], check=True)
        out = _run(_ORACLE_DRIVER, lib, asan, tmp)
        assert "oracle calls" in out


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_host_layer_under_asan_ubsan():
    rt = _clang_asan_runtime()
    objs = [os.path.join(PKG, "_build", n + ".o")
            for n in ("gdn_fwd.hip", "gdn_bwd.hip", "gdn_conv.hip")]
    if rt is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("clang's ASan runtime or the built kernel objects are missing")
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "sf_gdn_api.o")
        lib = os.path.join(tmp, "libsf_gdn.so")
        san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer"]
        subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                        "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
                       + san + ["-I", os.path.join(REPO, "include"), "-c",
                                os.path.join(PKG, "csrc", "sf_gdn_api.cpp"), "-o", obj],
                       check=True, capture_output=True)
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + san[:4]
                       + ["-shared-libasan", "-o", lib, obj] + objs, check=True,
                       capture_output=True)
        out = _run(_HOST_DRIVER, lib, rt, tmp)
        assert " passed" in out
