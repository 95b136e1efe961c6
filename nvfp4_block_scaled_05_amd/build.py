"""Build the gfx950 C-ABI library ``lib/libnvfp4.so`` in-tree with hipcc.

Usage: ``python -m nvfp4_block_scaled_05_amd.build`` (or ``build()``).  Every
call recompiles; the result is written to a temporary name and renamed, so a
concurrent loader never sees a half-written library.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libnvfp4.so")
PROBE_LIB = os.path.join(LIBDIR, "libnvfp4_probes.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled in generated code; divisions and square
# roots stay correctly rounded; no FP contraction, so the quantizer's binary32
# steps are exactly the written ones.
DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    "-I", INCLUDE, "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-I", INCLUDE, "-Wall"]

SOURCES = ["quantize.hip", "gemm_nvfp4.hip", "gemm.hip", "fp8.hip", "api.cpp"]
# test-only library: conversion probes and the calibration kernels of the
# roofline measurement (isa_probe.h, calib.h beside the sources)
PROBE_SOURCES = ["isa_probe.hip", "calib.hip"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    flags = DEVICE_FLAGS if src.endswith(".hip") else HOST_FLAGS
    cmd = [HIPCC, *flags, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(verbose=False):
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(5, len(srcs))) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    if verbose:
        for src, (_, out) in results.items():
            if out:
                print(f"[{src}]\n{out}")
    _link(LIB, [results[s][0] for s in SOURCES])
    _link(PROBE_LIB, [results[s][0] for s in PROBE_SOURCES])
    return LIB


def _link(target, objs):
    tmp = target + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, target)


def clean():
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
