"""Builds the library with AddressSanitizer on its host code only (device code is built as
usual) into _build/asan/liblwm_attn_asan.so, for the host-side boundary tests on the CPU.
Test infrastructure; no GPU run loads it."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

from long_context_exact_blockwise_amd import build as B

OUT_DIR = os.path.join(B.BUILD, "asan")
LIB = os.path.join(OUT_DIR, "liblwm_attn_asan.so")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libasan"]


def runtime() -> str | None:
    """The clang AddressSanitizer runtime that matches hipcc, to be preloaded into Python."""
    r = subprocess.run([B.HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
        return p
    base = "/opt/rocm/lib/llvm/lib/clang"
    if os.path.isdir(base):
        for v in sorted(os.listdir(base), reverse=True):
            cand = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(cand):
                return cand
    return None


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)

    def comp(src):
        obj = os.path.join(OUT_DIR, src + ".o")
        cmd = [B.HIPCC, *B.COMMON_FLAGS, *B.SOURCE_FLAGS.get(src, []), *HOST_ASAN]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        cmd += ["-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host ASan) failed for {src}:\n{r.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, B.SOURCES))
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_ASAN, "-o", LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host ASan) failed:\n{r.stderr}")
    return LIB
