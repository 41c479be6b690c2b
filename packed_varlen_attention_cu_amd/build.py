"""Build the in-tree shared library ``_lib/liblibra.so`` with hipcc for gfx950.

Usage: ``python -m packed_varlen_attention_cu_amd.build`` (or ``build_all()``):
builds ``_lib/liblibra.so`` and the counting build ``_lib/liblibra_debug.so``.
Every call compiles from source; nothing is cached.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "liblibra.so")
# The counting build: the forward kernel also counts the (query, key, head)
# triples it leaves unmasked (include/libra_debug.h); tests only.
DEBUG_LIB = os.path.join(LIBDIR, "liblibra_debug.so")
DEBUG_DEFINES = ("LIBRA_COUNT_PAIRS",)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["plan.cpp", "vrsp.cpp"]
DEVICE_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip"]
# Instruction scheduling per source, as measured: LLVM's max-ILP strategy makes
# the forward 3-5 % and the dQ pass up to 2 % faster but the dK/dV pass 3 %
# slower; the dK/dV pass keeps the default strategy (0.5-1 % ahead of the
# iterative max-occupancy one since its copies were made uniform).
SOURCE_FLAGS = {"attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
                "attn_bwd_dq.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}

COMMON = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-I", INCLUDE, "-I", CSRC, "-Wall"]
# Packed fp32 VALU forms are kept out of the generated code on purpose.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics",
                # keep MFMA accumulators in architectural VGPRs: the softmax works on them
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link ``out``; ``defines`` are extra -D macros."""
    libdir = os.path.dirname(os.path.abspath(out))
    os.makedirs(libdir, exist_ok=True)
    objdir = os.path.join(libdir, "obj_" + os.path.basename(out))
    shutil.rmtree(objdir, ignore_errors=True)
    os.makedirs(objdir)
    jobs = []
    for src in HOST_SOURCES:
        jobs.append([HIPCC, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, src),
                     "-o", os.path.join(objdir, src + ".o")])
    for src in DEVICE_SOURCES:
        jobs.append([HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *[f"-D{d}" for d in defines],
                     "-c", os.path.join(CSRC, src),
                     "-o", os.path.join(objdir, src + ".o")])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [os.path.join(objdir, s + ".o") for s in HOST_SOURCES + DEVICE_SOURCES]
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp])
    os.replace(tmp, out)
    shutil.rmtree(objdir, ignore_errors=True)
    return out


def build_all(verbose: bool = False):
    """The library and its counting build, compiled in parallel."""
    with ThreadPoolExecutor(2) as ex:
        jobs = [ex.submit(build, verbose), ex.submit(build, verbose, DEBUG_LIB, DEBUG_DEFINES)]
        return [j.result() for j in jobs]


if __name__ == "__main__":
    print(build_all(verbose=True))
