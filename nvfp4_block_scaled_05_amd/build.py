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
# api.cpp holds no device code: compiled for the host only
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "--cuda-host-only", "-I", INCLUDE, "-Wall"]

# The host-sanitizer build of the tests: the library's host code (argument
# checks, the layer predicate, launch set-up) under AddressSanitizer and
# UndefinedBehaviorSanitizer, each -fsanitize= behind -Xarch_host so no device
# code is instrumented.  Device code is compiled unoptimized: this build only
# runs where no GPU is present, so its kernels never execute.
SANITIZE_FLAGS = [
    "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
    "-I", INCLUDE,
]

SOURCES = ["quantize.hip", "gemm_nvfp4.hip", "gemm_nvfp4_quant.hip", "gemm.hip", "fp8.hip",
           "api.cpp"]
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
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
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


def asan_runtime():
    """Path of the AddressSanitizer runtime a process must preload to load the
    sanitizer build."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin",
                         "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_host_sanitized(outdir):
    """Build the library's sources with the sanitizer flags into
    ``outdir/libnvfp4_sanitized.so`` and return its path."""
    os.makedirs(outdir, exist_ok=True)

    def one(src):
        obj = os.path.join(outdir, src + ".o")
        cmd = [HIPCC, *SANITIZE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    target = os.path.join(outdir, "libnvfp4_sanitized.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-o", target] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer link failed:\n" + r.stdout + r.stderr)
    return target


def clean():
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
