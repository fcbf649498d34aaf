"""Float64 rotary position embedding (RoPE) with a large base theta, and attention on
rotated queries and keys.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source on the LWM pages (deep dive "LWM: million-token video-language world model"):
section "Stage I：长上下文语言模型" (stage I, long-context language model) says the context
is extended by enlarging RoPE's theta, and its Table 11 (and Table 13 of stage II) lists
theta per stage: 1M at 32K tokens, 10M at 128K and 256K, 25M at 512K, 50M at 1M.  The pages
give no formula; the reading used is the textbook rotary embedding of the LLaMA family:
head width D (even), pair i = (x[2i], x[2i+1]) for i = 0 .. D/2-1, frequency
    w_i = theta ** (-2 i / D),
and the vector of a token at position p has every pair rotated by the angle p * w_i:
    y[2i]   = x[2i] cos(p w_i) - x[2i+1] sin(p w_i)
    y[2i+1] = x[2i] sin(p w_i) + x[2i+1] cos(p w_i).
The inverse rotates by -p w_i; it is also the transpose, which is what carries a gradient
with respect to the rotated vector back to the unrotated one.  Positions are global token
positions (q_offset + i for query row i, k_offset + j for key j).  Because a rotated score
depends only on the difference of the two positions, and packed samples never attend
across their boundaries, global positions give the same attention as positions restarted
at every packed sample.
"""
from __future__ import annotations

import numpy as np

from . import attention as A


def frequencies(D: int, theta: float) -> np.ndarray:
    """w_i = theta^(-2i/D) for i = 0 .. D/2-1 (float64)."""
    if D % 2:
        raise ValueError("RoPE needs an even head width")
    return float(theta) ** (-np.arange(0, D, 2, dtype=np.float64) / D)


def rotate(x, positions, theta: float, inverse: bool = False):
    """Rotate the last axis (D) of x [..., S, D] for the S positions given (one per row of
    the second-to-last axis).  Returns float64."""
    x = np.asarray(x, np.float64)
    pos = np.asarray(positions, np.float64)
    ang = pos[:, None] * frequencies(x.shape[-1], theta)[None, :]  # [S, D/2]
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def attention_forward(q, k, v, seg_q, seg_k, scale, theta, causal=True, q_offset=0, k_offset=0):
    """(O, LSE) of attention on RoPE-rotated Q [B,H,Sq,D] and K [B,H,Sk,D]."""
    qr = rotate(q, q_offset + np.arange(q.shape[-2]), theta)
    kr = rotate(k, k_offset + np.arange(k.shape[-2]), theta)
    return A.forward(qr, kr, v, seg_q, seg_k, scale, causal, q_offset, k_offset)


def attention_backward(q, k, v, do, seg_q, seg_k, scale, theta, causal=True, q_offset=0,
                       k_offset=0):
    """(dQ, dK, dV) with respect to the unrotated Q and K: the gradient on the rotated
    vectors, rotated back (chain rule through the orthogonal rotation)."""
    qpos = q_offset + np.arange(q.shape[-2])
    kpos = k_offset + np.arange(k.shape[-2])
    qr, kr = rotate(q, qpos, theta), rotate(k, kpos, theta)
    dqr, dkr, dv = A.backward(qr, kr, v, do, seg_q, seg_k, scale, causal, q_offset, k_offset)
    return rotate(dqr, qpos, theta, inverse=True), rotate(dkr, kpos, theta, inverse=True), dv
