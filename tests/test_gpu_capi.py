"""The C-ABI used from C++ alone: tests/capi/capi_example (built by build() from
capi_example.cpp) reads inputs from files, calls lwm_attn_build_block_table, lwm_attn_fwd and
lwm_attn_bwd on a stream it creates, checks that a short workspace is refused, and writes its
outputs; they are compared here with the float64 oracle, every element."""
import math
import os
import subprocess

import numpy as np
import pytest

import lwm_inputs as li
from oracle import attention as A
import test_oracle_pins as pins
from gpu_helpers import TOL_LSE, TOL_O, check_grad, max_abs, say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "capi_example")


def test_capi_example_matches_oracle(tmp_path):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run build() first")
    B, H, S, D = 2, 2, 700, 128
    say(f"C-ABI example: B={B} H={H} S={S} D={D}")
    rng = np.random.default_rng(81)
    seg = np.stack([pins.random_layout(rng, S, allow_padding=(b == 1)) for b in range(B)]).astype(np.int32)
    bits = {n: li.bf16_bits_from_f32(li.host_normal((B, H, S, D), 81, 0.1 if n == "do" else 0.5, i))
            for i, n in enumerate(("q", "k", "v", "do"))}
    for n, b in bits.items():
        b.astype(np.uint16).tofile(tmp_path / f"{n}.bin")
    seg.tofile(tmp_path / "seg.bin")
    r = subprocess.run([EXE, str(B), str(H), str(S), str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    say(r.stdout.strip() or r.stderr.strip())
    assert r.returncode == 0, r.stderr
    rd = lambda n: li.bf16_bits_to_f64(np.fromfile(tmp_path / f"{n}.bin", np.uint16).reshape(B, H, S, D))
    o, dq, dk, dv = (rd(n) for n in ("o", "dq", "dk", "dv"))
    lse = np.fromfile(tmp_path / "lse.bin", np.float32).reshape(B, H, S).astype(np.float64)
    f = {n: li.bf16_bits_to_f64(b) for n, b in bits.items()}
    scale = 1 / math.sqrt(D)
    o_ref, lse_ref = A.forward(f["q"], f["k"], f["v"], seg, seg, scale)
    g_ref = A.backward(f["q"], f["k"], f["v"], f["do"], seg, seg, scale)
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    say(f"  max-abs O {eo:.2e} LSE {el:.2e}")
    assert np.array_equal(np.isinf(lse), np.isinf(lse_ref))
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE
    for n, g, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_ref):
        check_grad(n, g, ref, "bf16")
