"""Pure-Python loops over tiny inputs (no NumPy arithmetic).

TEST INFRASTRUCTURE ONLY.  These restate the definition in `oracle.attention` with scalar
loops and `math`, for S of a dozen tokens and D of a few lanes, so that the vectorised
oracle can be checked against an evaluation that shares none of its array code.
Inputs are nested Python lists: q[i][d], k[j][d], v[j][d], do[i][d]; seg_q[i], seg_k[j].
"""
from __future__ import annotations

import math


def _visible(seg_q, seg_k, i, j, q_offset, k_offset, causal):
    if seg_q[i] < 0 or seg_q[i] != seg_k[j]:
        return False
    return (not causal) or (k_offset + j <= q_offset + i)


def forward(q, k, v, seg_q, seg_k, scale, causal=True, q_offset=0, k_offset=0):
    """Returns (O as list of rows, LSE list); an empty row gives zeros and -inf."""
    Sq, Sk, D = len(q), len(k), len(v[0]) if v else 0
    out, lse = [], []
    for i in range(Sq):
        s = {}
        for j in range(Sk):
            if _visible(seg_q, seg_k, i, j, q_offset, k_offset, causal):
                dot = 0.0
                for d in range(len(q[i])):
                    dot += q[i][d] * k[j][d]
                s[j] = scale * dot
        if not s:
            out.append([0.0] * D)
            lse.append(-math.inf)
            continue
        m = max(s.values())
        den = 0.0
        for j in s:
            den += math.exp(s[j] - m)
        row = [0.0] * D
        for j in s:
            p = math.exp(s[j] - m) / den
            for d in range(D):
                row[d] += p * v[j][d]
        out.append(row)
        lse.append(m + math.log(den))
    return out, lse


def backward(q, k, v, do, seg_q, seg_k, scale, causal=True, q_offset=0, k_offset=0):
    """Returns (dQ, dK, dV) as lists of rows, from the softmax chain rule."""
    Sq, Sk, D = len(q), len(k), len(q[0])
    Dv = len(v[0])
    o, lse = forward(q, k, v, seg_q, seg_k, scale, causal, q_offset, k_offset)
    dq = [[0.0] * D for _ in range(Sq)]
    dk = [[0.0] * D for _ in range(Sk)]
    dv = [[0.0] * Dv for _ in range(Sk)]
    for i in range(Sq):
        if lse[i] == -math.inf:
            continue
        delta = 0.0
        for d in range(Dv):
            delta += do[i][d] * o[i][d]
        for j in range(Sk):
            if not _visible(seg_q, seg_k, i, j, q_offset, k_offset, causal):
                continue
            dot = 0.0
            for d in range(D):
                dot += q[i][d] * k[j][d]
            p = math.exp(scale * dot - lse[i])
            dp = 0.0
            for d in range(Dv):
                dp += do[i][d] * v[j][d]
                dv[j][d] += p * do[i][d]
            ds = p * (dp - delta)
            for d in range(D):
                dq[i][d] += scale * ds * k[j][d]
                dk[j][d] += scale * ds * q[i][d]
    return dq, dk, dv
