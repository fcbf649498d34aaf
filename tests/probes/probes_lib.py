"""Builds, loads and runs the gfx950 microbenchmarks of probes.hip (test infrastructure).

Each probe returns a rate measured with HIP events on torch's current stream:
  mfma    bf16 v_mfma_f32_32x32x16 throughput, TFLOP/s over the whole chip
  exp     v_exp_f32 wave instructions per second over the chip
  lds     LDS read bandwidth, bytes per second over the chip
  read    streaming read from HBM, bytes per second
  atomic  float32 atomic adds of 32 KiB tiles (the shape of a query tile's dQ), bytes per second
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "probes.hip")
LIB = os.path.join(HERE, "liblwm_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    r = subprocess.run([HIPCC, *FLAGS, SRC, "-o", LIB + ".tmp"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probes.hip:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built")
        _lib = ctypes.CDLL(LIB)
        I, P, I64 = ctypes.c_int, ctypes.c_void_p, ctypes.c_int64
        for name, args in (("lwm_probe_mfma", [I, I, P, P]), ("lwm_probe_exp", [I, I, P, P]),
                           ("lwm_probe_lds", [I, I, P, P]), ("lwm_probe_read", [I, P, I64, P, P]),
                           ("lwm_probe_atomic", [I, P, I64, I, P]),
                           ("lwm_probe_mfma16_layout", [P, P, P, P])):
            fn = getattr(_lib, name)
            fn.restype, fn.argtypes = I, args
    return _lib


def _time(torch, fn, reps=3):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3  # seconds


def run(torch, scale: float = 1.0) -> dict:
    """All probes; `scale` shortens them (the GPU test runs them small)."""
    lib = load()
    st = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"cus": cus}
    blocks = cus * 4
    # one float per thread of the largest grid below (the read probe's blocks * 4)
    sink = torch.empty(blocks * 4 * 256, dtype=torch.float32, device="cuda")
    chk = lambda rc: (_ for _ in ()).throw(RuntimeError(f"probe launch failed: {rc}")) if rc else None

    it = max(1, int(65536 * scale))  # about 4 ms per launch: long enough to meet the power limit
    s = _time(torch, lambda: chk(lib.lwm_probe_mfma(blocks, it, sink.data_ptr(), st)))
    out["mfma_bf16_tflops"] = blocks * 4 * it * 4 * 32768 / s / 1e12

    it = max(1, int(65536 * scale))
    s = _time(torch, lambda: chk(lib.lwm_probe_exp(blocks, it, sink.data_ptr(), st)))
    out["exp_wave_instr_per_s"] = blocks * 4 * it * 8 / s
    out["exp_cycles_per_instr_per_simd_at_2.4GHz"] = (cus * 4) * 2.4e9 / out["exp_wave_instr_per_s"]

    it = max(1, int(16384 * scale))
    s = _time(torch, lambda: chk(lib.lwm_probe_lds(blocks, it, sink.data_ptr(), st)))
    out["lds_read_bytes_per_s"] = blocks * 256 * it * 16 * 16 / s
    out["lds_read_bytes_per_clk_per_cu_at_2.4GHz"] = out["lds_read_bytes_per_s"] / cus / 2.4e9

    nbytes = int((8 << 30) * scale) // 16 * 16
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = _time(torch, lambda: chk(lib.lwm_probe_read(blocks * 4, src.data_ptr(), nbytes // 16, sink.data_ptr(), st)))
    out["hbm_read_bytes_per_s"] = nbytes / s
    del src

    ntiles = 65536 if scale >= 1 else 4096
    steps = max(1, int(64 * scale))
    dst = torch.zeros(ntiles * 8192, dtype=torch.float32, device="cuda")
    nb = 2048
    s = _time(torch, lambda: chk(lib.lwm_probe_atomic(nb, dst.data_ptr(), ntiles, steps, st)))
    out["atomic_add_f32_bytes_per_s"] = nb * steps * 8192 * 4 / s
    out["atomic_pattern"] = (f"{nb} workgroups x {steps} tiles of 64 x 128 float32 (32 KiB), "
                             f"workgroup w at step t on tile (w + t) mod {ntiles}")
    del dst
    return out


def mfma16_layout_ok(torch) -> bool:
    """Integer matrices (exact in bf16 and float32) through one 16x16x32 MFMA in the assumed
    operand layout, against torch's float64 product on the CPU."""
    lib = load()
    g = torch.Generator().manual_seed(5)
    A = torch.randint(-8, 9, (16, 32), generator=g).float()
    B = torch.randint(-8, 9, (32, 16), generator=g).float()
    Ad, Bd = A.cuda(), B.cuda()
    C = torch.full((16, 16), float("nan"), device="cuda")
    rc = lib.lwm_probe_mfma16_layout(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    if rc:
        raise RuntimeError(f"probe launch failed: {rc}")
    torch.cuda.synchronize()
    return bool(torch.equal(C.cpu().double(), A.double() @ B.double()))
