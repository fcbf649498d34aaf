"""Build liblwm_attn.so for gfx950 in-tree with hipcc.

Usage: python -m long_context_exact_blockwise_amd.build   (or call build()).
Every HIP source is compiled for gfx950 only; packed-FP32 instruction selection is turned
off for device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblwm_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "table.hip", "attn_f32.hip", "attn_bf16.hip", "merge.hip", "rope.hip",
           "packed_loss.hip", "decode_noalloc.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# attn_bf16.hip: MFMAs in the VGPR form, so that score accumulators feed the softmax without
# AGPR copies; the dK/dV kernel keeps its accumulators in AGPRs through asm constraints.
SOURCE_FLAGS = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# The race-canary build: the bf16 attention kernels with a wait and a workgroup barrier after
# every phase of a tile step (LWM_RACE_CANARY), linked into a library of its own that the GPU
# tests compare bit for bit with the normal one.
CANARY_LIB = os.path.join(PKG, "liblwm_attn_canary.so")
CANARY_SOURCES = {"attn_bf16.hip": ["-DLWM_RACE_CANARY"]}
# Every source again with the device checks of LWM_DEBUG (indices derived from the block table
# checked against the extents they index, failures recorded on the device and read back by
# lwm_attn_debug_status), linked into a third library for the tests.
DEBUG_LIB = os.path.join(PKG, "liblwm_attn_debug.so")
DEBUG_FLAGS = ["-DLWM_DEBUG"]


def _compile(src: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + suffix + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


# The compiler the GPU parity suite was last run green with.  The dK/dV kernel's
# accumulations are inline-asm MFMAs whose hazard wait states are written into the asm, which
# the compiler's hazard checks do not see; a different compiler may place its own code between
# them differently, so after a toolchain change the GPU gradient tests must pass again before
# the library is used.
VALIDATED_COMPILER = "AMD clang version 22.0.0git (https://github.com/RadeonOpenCompute/llvm-project roc-7.2.0 26014 7b800a19466229b8479a78de19143dc33c3ab9b5)"


def compiler_version() -> str:
    r = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    for line in r.stdout.splitlines():
        if "clang version" in line:
            return line.strip()
    return r.stdout.strip()


def build(verbose: bool = False) -> str:
    """Compile every source, link the shared library, its race-canary twin and its build with
    device checks; returns the library's path."""
    seen = compiler_version()
    if seen != VALIDATED_COMPILER:
        print(f"WARNING: building with\n  {seen}\nbut the GPU parity suite was validated with\n  "
              f"{VALIDATED_COMPILER}\nrun `pytest tests -m gpu` before using this build (the dK/dV "
              "kernel's asm MFMAs carry hand-written hazard waits)", file=sys.stderr, flush=True)
    os.makedirs(BUILD, exist_ok=True)
    n = len(SOURCES)
    jobs = [(src, (), "") for src in SOURCES]
    jobs += [(src, tuple(DEBUG_FLAGS), ".debug") for src in SOURCES]
    jobs += [(src, tuple(flags), ".canary") for src, flags in CANARY_SOURCES.items()]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    normal, debug = objs[:n], objs[n:2 * n]
    canary = [o for o in normal]
    for (src, _, _), o in zip(jobs[2 * n:], objs[2 * n:]):
        canary[SOURCES.index(src)] = o
    _link(normal, LIB)
    _link(canary, CANARY_LIB)
    _link(debug, DEBUG_LIB)
    if verbose:
        print(f"built {LIB}, {CANARY_LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
