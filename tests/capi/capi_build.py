"""Builds tests/capi/capi_example (a C++ program calling the library's C-ABI only), linked
against the in-tree liblwm_attn.so with an rpath to it.  Test infrastructure."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "long_context_exact_blockwise_amd")
EXE = os.path.join(HERE, "capi_example")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "capi_example.cpp"), "-o", EXE + ".tmp", "-L", PKG, "-llwm_attn",
           f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for capi_example.cpp:\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
