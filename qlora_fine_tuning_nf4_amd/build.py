"""Build the HIP library in-tree: ``python -m qlora_fine_tuning_nf4_amd.build``.

Compiles every source under ``csrc/`` for gfx950 with hipcc into
``qlora_fine_tuning_nf4_amd/libqlora_nf4.so`` (one object per source, then one
shared link), so the built library travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqlora_nf4.so")
# the benchmark's measured-ceiling probes, a library of their own
PEAKS_SRC = "peaks.hip"
PEAKS_OUT = os.path.join(HERE, "libqlora_peaks.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "gemv.hip", "lora.hip", "scratch.hip",
           "relayout.hip"]

ARCH = os.environ.get("QLORA_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 VALU forms stay off (the plain scalar forms are used instead)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    # a failed build must not leave an older library behind
    for out in (OUT, PEAKS_OUT):
        if os.path.exists(out):
            os.remove(out)
    srcs = SOURCES + [PEAKS_SRC]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], OUT)
    _link(objs[-1:], PEAKS_OUT)
    if verbose:
        print(f"built {OUT} and {PEAKS_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
