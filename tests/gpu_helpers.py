"""Helpers shared by the GPU parity tests: device transfer of seeded inputs and read-back
of results as float64.  Holds no attention arithmetic."""
from __future__ import annotations

import sys

import numpy as np

import lwm_inputs as li

# Tolerances stated for this path: O max-abs 1e-2 (bf16 inputs) / 2e-5 (fp32 inputs),
# LSE max-abs 1e-3.  Gradients are held to the same max-abs bars as O and, since gradients
# are small at these input scales (dO ~ N(0,1) * 0.1), also to relative bars: max-abs over
# max |ref| and the relative Frobenius error.  bf16: P and dS are rounded to bf16 before the
# gradient products and the results are rounded once more, each a relative error of at most
# 2^-9, so errors of a few 1e-3 are expected; the bars leave about 2.5x margin.
TOL_O = {"bf16": 1e-2, "f32": 2e-5}
TOL_LSE = 1e-3
TOL_GRAD = {"bf16": 1e-2, "f32": 2e-5}
TOL_GRAD_RELMAX = {"bf16": 2e-2, "f32": 1e-4}
TOL_GRAD_RELFRO = {"bf16": 1e-2, "f32": 1e-4}


def say(*a):
    """Print and flush, so a log names the case that was running."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype_name):
    """numpy (float32 values or uint16 bf16 bits) -> contiguous CUDA tensor."""
    import torch

    if dtype_name == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda().contiguous()


def seg_dev(seg):
    import torch

    return torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).cuda().contiguous()


def f64(t):
    """CUDA tensor -> float64 numpy (exact for bf16 and fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_f64(arr, dtype_name):
    return li.bf16_bits_to_f64(arr) if dtype_name == "bf16" else np.asarray(arr, np.float64)


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):  # inf - inf on the pairs both_inf excludes
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d))


def rel_errors(got, ref):
    """(max-abs / max-|ref|, relative Frobenius error) of a gradient, both reported beside
    the max-abs bar."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    mref = float(np.max(np.abs(r))) if r.size else 0.0
    nref = float(np.linalg.norm(r))
    mabs = float(np.max(np.abs(g - r))) if r.size else 0.0
    return (mabs / mref if mref > 0 else 0.0), (float(np.linalg.norm(g - r)) / nref if nref > 0 else 0.0)


def check_grad(name, got, ref, dt):
    """Assert the max-abs and both relative bars on one gradient; returns the three errors."""
    g = np.asarray(got, np.float64)
    ea = max_abs(g, ref)
    rm, rf = rel_errors(g, ref)
    say(f"  {name}: max-abs {ea:.2e}, max-abs/max-ref {rm:.2e}, rel Frobenius {rf:.2e}")
    assert ea <= TOL_GRAD[dt], (name, ea)
    # a reference that is zero up to rounding (one key per row, Q = 0 dK) has no scale to be
    # relative to; the max-abs bar alone applies there
    if np.size(ref) and float(np.max(np.abs(ref))) > 1e-6:
        assert rm <= TOL_GRAD_RELMAX[dt], (name, rm)
        assert rf <= TOL_GRAD_RELFRO[dt], (name, rf)
    return ea, rm, rf
