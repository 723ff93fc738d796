"""Build libmsa.so (host runtime + gfx950 kernels) in-tree with hipcc.

    python -m kv_cache_attention_msa_amd.csrc.build                # or build() from Python
    python -m kv_cache_attention_msa_amd.csrc.build --phase-trace  # measurement build

Every call compiles every source again (objects go to ``_build/`` at the
repository root, the library to ``kv_cache_attention_msa_amd/libmsa.so``).
``--phase-trace`` builds ``libmsa_trace.so`` instead: the same library with
MSA_PHASE_TRACE defined, whose chunk kernel records per-phase clocks
(``bench.py --phase-trace``); it is never loaded unless asked for.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")
TRACE_LIB = os.path.join(PKG, "libmsa_trace.so")   # measurement build (MSA_PHASE_TRACE)
PEAKS_LIB = os.path.join(PKG, "libmsa_peaks.so")   # measurement probes (benchmark only)
PEAKS_SOURCE = os.path.join(HERE, "peaks", "msa_peaks.hip")
ARCH = "gfx950"

HOST_SOURCES = ["msa_plan.cpp", "msa_api.cpp", "msa_latency.cpp", "msa_evict.cpp"]
HIP_SOURCES = sorted(f for f in os.listdir(HERE) if f.endswith(".hip"))

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{HERE}", "-Wall", "-Wno-unused-function"]
COMMON += os.environ.get("MSA_EXTRA_CFLAGS", "").split()  # extra compiler flags (tuning experiments)
# Packed fp32 ops stay off: the kernels are written for scalar fp32 VALU math.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]
# The bf16 attention kernels never feed NaN into their max/exp arithmetic (pool
# slots outside the segments are selected out or zeroed), so max needs no
# NaN canonicalisation there.
NO_NAN_SOURCES = {"msa_prefill.hip", "msa_decode.hip"}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def _build_lib(lib: str, objdir: str, defines, verbose: bool, jobs: int) -> None:
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    cmds, objs = [], []
    for src in HOST_SOURCES + HIP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        extra = DEVICE + ["-x", "hip"] if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"]
        if src in NO_NAN_SOURCES:
            extra = ["-fno-honor-nans"] + extra
        cmds.append([cc, "-c"] + COMMON + list(defines) + extra + [os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for c, o in zip(cmds, outs):
            print(" ".join(c))
            if o.strip():
                print(o)
    tmp = lib + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, lib)


def build_trace(verbose: bool = False, jobs: int = 8) -> str:
    """The measurement build: libmsa_trace.so with MSA_PHASE_TRACE."""
    _build_lib(TRACE_LIB, os.path.join(BUILD, "trace"), ["-DMSA_PHASE_TRACE"], verbose, jobs)
    return TRACE_LIB


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    _build_lib(LIB, BUILD, [], verbose, jobs)
    tmp = PEAKS_LIB + ".tmp"
    _run([cc, "-shared"] + COMMON + DEVICE + ["-x", "hip", PEAKS_SOURCE, "-o", tmp])
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    if "--phase-trace" in sys.argv:
        print(build_trace(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
