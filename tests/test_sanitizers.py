"""The oracle and the library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
in CPU builds: the oracle (gcc) runs every reconstruction, calibration, tail policy and gradient mode
with flags and flips on ragged sizes; the library's host side (hipcc, host code only) runs its
argument checks, layouts and error paths.  Each run is a child process with the sanitizer runtime
preloaded; any report fails the test."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_softmax_attention_kia_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

ORACLE_SCRIPT = r'''
import itertools, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
from oracle import oracle as ORC
rng = np.random.default_rng(5)
cases = []
for recon in ("lerp", "nearest", "binmean", "nearest_binmean"):
    for calib, tail in (("minmax", "zero"), ("fwm", "zero"), ("fwm", "floor"), ("fwm", "resolved")):
        if recon in ("binmean", "nearest_binmean") and tail != "zero":
            continue
        for ste, grad in (("weight", "full"), ("prob", "full"), ("prob", "detached"), ("prob", "max_only"),
                          ("prob", "min_only"), ("prob", "p1")):
            cases.append(ORC.OracleConfig(calib, recon, ste, grad, 4, 3.0, tail=tail))
for recon in ("softmax", "exp_bf16", "exp_fp8"):
    for grad in ("full", "detached", "p1"):
        cases.append(ORC.OracleConfig("fwm", recon, "prob", grad, 4))
cases.append(ORC.OracleConfig("minmax", "lerp", "prob", "full", 64))
cases.append(ORC.OracleConfig("minmax", "lerp", "prob", "full", 1))
n = 0
for cfg in cases:
    for T, D, causal in ((37, 16, True), (1, 8, True), (20, 8, False)):
        q, k, v, do = (rng.standard_normal((T, D)).astype(np.float32).astype(np.float64) for _ in range(4))
        k[3 % T] = k[0]                     # tied keys: tied extrema in some rows
        ref = ORC.head(cfg, q, k, v, do, causal=causal, guard=1e-3, flag_cap=4096, bins=True)
        fl = ref["flags"][:8]
        if len(fl):
            ORC.head(cfg, q, k, v, do, causal=causal, rows=sorted({int(r) for r in fl[:, 0]}), flips=fl, nthreads=1)
        flat = np.zeros((T, D))
        ORC.head(cfg, flat, flat, v, do, causal=causal)
        s = rng.standard_normal(T) * 3
        ORC.row(cfg, s, rng.standard_normal(T), flip=np.full(T, 127, np.uint8))
        n += 1
print("oracle runs", n)
'''

HOST_SCRIPT = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from quantized_softmax_attention_kia_amd import binding as kb
lib = kb.load_library(sys.argv[2])
P = kb.Params
def params(**kw):
    base = dict(B=2, H=3, T=100, D=64, causal=1, K=4, tau=8.0, scale=0.125, calib=0, recon=0, ste=0, grad=0,
                dtype=0, tail=0)
    base.update(kw)
    return P(**base)
a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
n = 0
for calib in (0, 1):
    for recon in range(7):
        for ste in (0, 1):
            for grad in range(5):
                for tail in (0, 1, 2):
                    for dtype in (0, 1):
                        for T, D, K in ((100, 64, 4), (1, 128, 64), (0, 64, 1), (33, 48, 4), (-1, 64, 4)):
                            p = params(calib=calib, recon=recon, ste=ste, grad=grad, tail=tail, dtype=dtype,
                                       T=T, D=D, K=K)
                            lib.kia_workspace_size(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b))
                            n += 1
bad = [dict(K=0), dict(K=65), dict(D=48), dict(T=-1), dict(calib=1, tau=0.0), dict(calib=1, tau=float("nan")),
       dict(recon=9), dict(ste=-1), dict(grad=5), dict(dtype=7), dict(causal=2), dict(scale=-1.0),
       dict(scale=float("inf")), dict(B=-1), dict(recon=5, K=9), dict(calib=0, tail=2)]
for kw in bad:
    p = params(**kw)
    st = lib.kia_forward(ctypes.byref(p), None, None, None, None, None, None)
    assert st != 0, kw
    assert lib.kia_backward(ctypes.byref(p), *([None] * 11)) != 0
    assert lib.kia_backward_noalloc(ctypes.byref(p), *([None] * 10)) != 0
    assert lib.kia_debug_bins(ctypes.byref(p), None, None, None) != 0
    assert lib.kia_flash_forward(ctypes.byref(p), None, None, None, None, None, None) != 0
    assert lib.kia_forward_scores(ctypes.byref(p), None, None, None, None, None) != 0
    assert lib.kia_forward_weights(ctypes.byref(p), None, None, None, None, None, None) != 0
    assert lib.kia_flash_backward(ctypes.byref(p), *([None] * 10)) != 0
    lib.kia_last_error()
# the one-pass kernels compute softmax only; null buffers are rejected
assert lib.kia_flash_forward(ctypes.byref(params()), None, None, None, None, None, None) == -2
assert lib.kia_flash_forward(ctypes.byref(params(recon=2, calib=1)), None, None, None, None, None, None) == -1
assert lib.kia_flash_backward(ctypes.byref(params(recon=2, calib=1)), *([None] * 10)) == -1
# valid params, null buffers: rejected before any launch
p = params()
assert lib.kia_forward(ctypes.byref(p), None, None, None, None, None, None) != 0
assert lib.kia_backward(ctypes.byref(p), *([None] * 11)) != 0
# the built-in workspace is too small for these: rejected before any device call
p = params(B=4, H=16, T=1024)
assert lib.kia_backward_noalloc(ctypes.byref(p), *([None] * 10)) == -3
for s in range(-6, 2):
    lib.kia_status_string(s)
# empty problems: nothing to do
p = params(B=0)
assert lib.kia_forward(ctypes.byref(p), None, None, None, None, None, None) == 0
print("host calls", n)
'''


def _run(script, env, *args):
    r = subprocess.run([sys.executable, "-c", script, ROOT, *args], env=env, capture_output=True, text=True,
                       timeout=600)
    report = r.stderr[-4000:]
    assert r.returncode == 0 and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libkia_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-o", lib, os.path.join(ROOT, "oracle", "kia_oracle.c"), "-lm"])
    env = dict(os.environ, KIA_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    out = _run(ORACLE_SCRIPT, env)
    assert "oracle runs" in out


def test_host_code_under_asan_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(HIPCC) or not os.path.exists(CLANGXX):
        pytest.skip("the ROCm toolchain or its AddressSanitizer runtime is not installed")
    # the C ABI (argument checks, layouts, error paths) with host-side sanitizers; the kernel
    # dispatchers are test-only stand-ins, never reached (every call here is rejected before a launch)
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "api.o")
    stubs = str(tmp_path / "stubs.o")
    subprocess.check_call([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", *san, *inc, "-c",
                           os.path.join(CSRC, "kia_api.hip"), "-o", api], stderr=subprocess.DEVNULL)
    subprocess.check_call([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *san, *inc,
                           "-c", os.path.join(ROOT, "tests", "sanitizer_stubs.cpp"), "-o", stubs],
                          stderr=subprocess.DEVNULL)
    objs = [api, stubs]
    lib = str(tmp_path / "libkia_host_san.so")
    hip_lib = "/opt/rocm/lib"
    subprocess.check_call([CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", "-o", lib,
                           *objs, f"-L{hip_lib}", "-lamdhip64", f"-Wl,-rpath,{hip_lib}"])
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run(HOST_SCRIPT, env, lib)
    assert "host calls" in out
