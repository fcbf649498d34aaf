"""The gfx950 microbenchmarks (tests/probes) run briefly and report rates in the range the
part's specification allows: they back the chip facts the kernel design rests on, and
`python bench.py --probes` runs them at full length."""
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes"))

from gpu_helpers import say  # noqa: E402


def test_probes_report_rates_within_the_specification():
    import probes_lib

    r = probes_lib.run(torch, scale=0.125)
    say("probes: " + ", ".join(f"{k} {v:.3g}" if isinstance(v, float) else f"{k} {v}" for k, v in r.items()))
    assert 200 < r["mfma_bf16_tflops"] < 2600          # published dense peak 2.5 PFLOP/s
    assert 0 < r["exp_wave_instr_per_s"]
    assert 1e12 < r["lds_read_bytes_per_s"]
    assert 5e11 < r["hbm_read_bytes_per_s"] < 8.2e12   # published HBM3E peak 8 TB/s
    assert 1e10 < r["atomic_add_f32_bytes_per_s"]


def test_mfma_16x16x32_operand_layout():
    """The operand and result lane layout of v_mfma_f32_16x16x32_bf16 that the kernels
    assume, checked with integer matrices against a host product."""
    import probes_lib

    assert probes_lib.mfma16_layout_ok(torch)
