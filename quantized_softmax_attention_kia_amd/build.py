"""Build libkia.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m quantized_softmax_attention_kia_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkia.so")
# (source, object, defines): the forward and dq kernels are built once per calibration
# (MinMax, FWM with a zero, floored or resolved tail, the exponential baselines); the KIA_CAL=0
# backward build also holds the dkdv kernel
NCALIB = 5
SOURCES = [("kia_api.hip", "kia_api.o", []), ("kia_flash.hip", "kia_flash.o", [])] + [
    (src, f"{src[:-4]}_c{c}.o", [f"-DKIA_CAL={c}"]) for c in range(NCALIB) for src in ("kia_fwd.hip", "kia_bwd.hip")]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str, defines) -> None:
    cmd = [HIPCC, *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")


def build(verbose: bool = True) -> str:
    with tempfile.TemporaryDirectory(prefix="kia_build_") as tmp:
        objs = [os.path.join(tmp, o) for _, o, _ in SOURCES]
        jobs = [(src, obj, d) for (src, _, d), obj in zip(SOURCES, objs)]
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda j: _compile(*j), jobs))
        out = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
