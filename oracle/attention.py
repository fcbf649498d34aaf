"""Float64 definition of masked causal softmax attention and its gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function forms the full masked
score matrix, or whole rows of it, and evaluates the definition below directly; there is no
blocking, tiling or online rescaling here.

Sources on the LWM pages (deep dive "LWM: million-token video-language world model"):
  * exact full attention, no window or sparse approximation: section "RingAttention 为什么
    必要" (why RingAttention is necessary), first list item;
  * causal next-token model over one token sequence: sections "核心问题" (core problem)
    and "模型结构" (model structure, table row "Training objective");
  * packed samples only see themselves: section "Masked sequence packing", first step.
The pages print no formula; the reading used (plain softmax attention, scale given by the
caller, natural-log LSE, empty rows give O = 0 and LSE = -inf) is the textbook one.

Definition, for one (batch, head), query row i at global position q_offset + i and key j
at global position k_offset + j:
  visible(i, j) = seg_q[i] >= 0 and seg_q[i] == seg_k[j] and
                  (not causal or k_offset + j <= q_offset + i)
  s_ij  = scale * <q_i, k_j>
  m_i   = max over visible j of s_ij
  l_i   = sum over visible j of exp(s_ij - m_i)
  P_ij  = exp(s_ij - m_i) / l_i on visible pairs, 0 elsewhere
  O_i   = sum_j P_ij v_j,      LSE_i = m_i + ln l_i
Gradient of the same map for an upstream dO (chain rule through softmax):
  dV_j = sum_i P_ij dO_i,  dP_ij = <dO_i, v_j>,  Delta_i = <dO_i, O_i>,
  dS_ij = P_ij (dP_ij - Delta_i),  dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i
A backward that is handed the forward's stored output O' (rounded to the storage dtype) forms
Delta_i = <dO_i, O'_i> from it; with c_i = <dO_i, O'_i - O_i> held fixed its dQ, dK are the
exact gradients of sum_i <dO_i, O_i> - sum_i c_i LSE_i (d LSE_i / d s_ij = P_ij), and dV is
unchanged.  backward(..., o=O') evaluates that; o=None uses the exact O.
Partial state over a subset C of keys (a KV chunk), relative to a reference max m:
  m = max over visible j in C of s_ij,  l = sum exp(s_ij - m),  acc = sum exp(s_ij - m) v_j
  empty subset: (m, l, acc) = (-inf, 0, 0)
"""
from __future__ import annotations

import numpy as np

EMPTY_M = -np.inf


def visibility(seg_q, seg_k, q_offset: int = 0, k_offset: int = 0, causal: bool = True):
    """Boolean [Sq, Sk] mask of visible (query, key) pairs for one batch row."""
    seg_q = np.asarray(seg_q)
    seg_k = np.asarray(seg_k)
    m = (seg_q[:, None] >= 0) & (seg_q[:, None] == seg_k[None, :])
    if causal:
        qpos = q_offset + np.arange(seg_q.shape[0], dtype=np.int64)
        kpos = k_offset + np.arange(seg_k.shape[0], dtype=np.int64)
        m &= kpos[None, :] <= qpos[:, None]
    return m


def _masked_scores(q, k, mask, scale):
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    return np.where(mask, s, -np.inf)


def _softmax_parts(s_masked):
    """Row max, exp(s - max) on visible entries (0 elsewhere) and row sums; empty rows keep
    m = -inf, e = 0, l = 0 without forming (-inf) - (-inf)."""
    m = s_masked.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.where(np.isfinite(s_masked), np.exp(s_masked - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    return m, e, l


def forward_head(q, k, v, mask, scale):
    """(O [Sq,D], LSE [Sq], P [Sq,Sk]) for one head.  Empty rows: O = 0, LSE = -inf."""
    s = _masked_scores(q, k, mask, scale)
    m, e, l = _softmax_parts(s)
    nonempty = l > 0
    p = np.where(nonempty[:, None], e / np.where(nonempty, l, 1.0)[:, None], 0.0)
    o = p @ np.asarray(v, np.float64)
    lse = np.where(nonempty, m + np.log(np.where(nonempty, l, 1.0)), -np.inf)
    return o, lse, p


def backward_head(q, k, v, do, mask, scale, o=None):
    """(dQ, dK, dV) for one head, float64.  o: the stored forward output Delta is formed
    from (None: the exact output)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    o_exact, _, p = forward_head(q, k, v, mask, scale)
    o = o_exact if o is None else np.asarray(o, np.float64)
    dv = p.T @ do
    dp = do @ v.T
    delta = (do * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def forward(q, k, v, seg_q, seg_k, scale, causal=True, q_offset=0, k_offset=0):
    """Batched forward over [B,H,Sq,D] / [B,H,Sk,D] with seg [B,S]; returns (O, LSE)."""
    B, H, Sq, D = q.shape
    o = np.zeros((B, H, Sq, D), np.float64)
    lse = np.zeros((B, H, Sq), np.float64)
    for b in range(B):
        mask = visibility(seg_q[b], seg_k[b], q_offset, k_offset, causal)
        for h in range(H):
            o[b, h], lse[b, h], _ = forward_head(q[b, h], k[b, h], v[b, h], mask, scale)
    return o, lse


def backward(q, k, v, do, seg_q, seg_k, scale, causal=True, q_offset=0, k_offset=0, o=None):
    """Batched gradient; returns (dQ, dK, dV) in float64.  o [B,H,Sq,D]: the stored forward
    output the backward is handed (None: the exact output)."""
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    for b in range(q.shape[0]):
        mask = visibility(seg_q[b], seg_k[b], q_offset, k_offset, causal)
        for h in range(q.shape[1]):
            args = (q[b, h], k[b, h], v[b, h], do[b, h], mask, scale)
            dq[b, h], dk[b, h], dv[b, h] = (backward_head(*args) if o is None
                                            else backward_head(*args, o=o[b, h]))
    return dq, dk, dv


def partial_state(q, k, v, mask, scale):
    """(m [Sq], l [Sq], acc [Sq,D]) of one head over the keys given (one KV chunk)."""
    s = _masked_scores(q, k, mask, scale)
    m, e, l = _softmax_parts(s)
    acc = e @ np.asarray(v, np.float64)
    return m, l, acc


def merge_states(a, b):
    """Combine two partial states over disjoint key sets into the state over their union:
    m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), acc likewise.  An empty side
    (m = -inf, l = 0) contributes nothing; two empty sides give an empty state."""
    m1, l1, acc1 = a
    m2, l2, acc2 = b
    m = np.maximum(m1, m2)
    both_empty = ~np.isfinite(m)
    m_safe = np.where(both_empty, 0.0, m)
    w1 = np.where(np.isfinite(m1), np.exp(np.where(np.isfinite(m1), m1, 0.0) - m_safe), 0.0)
    w2 = np.where(np.isfinite(m2), np.exp(np.where(np.isfinite(m2), m2, 0.0) - m_safe), 0.0)
    l = l1 * w1 + l2 * w2
    acc = acc1 * w1[:, None] + acc2 * w2[:, None]
    return np.where(both_empty, -np.inf, m), l, acc


def finalize_state(state):
    """(O, LSE) from a partial state: O = acc / l, LSE = m + ln l; empty rows O = 0, -inf."""
    m, l, acc = state
    nonempty = l > 0
    o = np.where(nonempty[:, None], acc / np.where(nonempty, l, 1.0)[:, None], 0.0)
    lse = np.where(nonempty, m + np.log(np.where(nonempty, l, 1.0)), -np.inf)
    return o, lse


def forward_rows(q_rows, k, v, seg_rows, seg_k, row_pos, scale, causal=True, k_offset=0,
                 strip=16):
    """Forward for selected query rows of one head: q_rows [R,D], their global positions
    row_pos [R] and segment ids seg_rows [R], against all keys k, v [Sk,D].  Each row's full
    masked score row is formed; rows are processed `strip` at a time to bound memory."""
    q_rows = np.asarray(q_rows, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    seg_k = np.asarray(seg_k)
    kpos = k_offset + np.arange(k.shape[0], dtype=np.int64)
    R = q_rows.shape[0]
    o = np.zeros((R, k.shape[1] if v.ndim == 2 else 0), np.float64)
    lse = np.zeros(R, np.float64)
    for s0 in range(0, R, strip):
        sl = slice(s0, min(R, s0 + strip))
        sq = np.asarray(seg_rows)[sl]
        mask = (sq[:, None] >= 0) & (sq[:, None] == seg_k[None, :])
        if causal:
            mask &= kpos[None, :] <= np.asarray(row_pos)[sl][:, None]
        o[sl], lse[sl], _ = forward_head(q_rows[sl], k, v, mask, scale)
    return o, lse


def dq_rows(q_rows, k, v, do_rows, seg_rows, seg_k, row_pos, scale, causal=True, k_offset=0,
            strip=16):
    """dQ for selected query rows of one head.  dQ_i depends only on row i's own softmax:
    dQ_i = scale * sum_j P_ij (<dO_i, v_j> - <dO_i, O_i>) k_j, with O_i from the same row."""
    q_rows = np.asarray(q_rows, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do_rows = np.asarray(do_rows, np.float64)
    seg_k = np.asarray(seg_k)
    kpos = k_offset + np.arange(k.shape[0], dtype=np.int64)
    R = q_rows.shape[0]
    dq = np.zeros_like(q_rows)
    for s0 in range(0, R, strip):
        sl = slice(s0, min(R, s0 + strip))
        sq = np.asarray(seg_rows)[sl]
        mask = (sq[:, None] >= 0) & (sq[:, None] == seg_k[None, :])
        if causal:
            mask &= kpos[None, :] <= np.asarray(row_pos)[sl][:, None]
        o, _, p = forward_head(q_rows[sl], k, v, mask, scale)
        dp = do_rows[sl] @ v.T
        delta = (do_rows[sl] * o).sum(axis=1)
        ds = p * (dp - delta[:, None])
        dq[sl] = scale * (ds @ k)
    return dq
