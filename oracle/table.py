"""Exact classification of (query block, key block) tile pairs.

TEST INFRASTRUCTURE ONLY.  A tile pair is SKIP when none of its (query, key) pairs is
visible, FULL when it lies wholly inside [0,Sq) x [0,Sk) and every pair is visible, and
PARTIAL otherwise.  Derived by reducing the visibility mask of `oracle.attention`, i.e. by
brute force over every pair; the codes are the ones the library's block table uses.
"""
from __future__ import annotations

import numpy as np

from .attention import visibility

SKIP, PARTIAL, FULL = 0, 1, 2


def classify(seg_q, seg_k, block_q, block_k, q_offset=0, k_offset=0, causal=True):
    """uint8 [ceil(Sq/block_q), ceil(Sk/block_k)] status matrix for one batch row."""
    mask = visibility(seg_q, seg_k, q_offset, k_offset, causal)
    Sq, Sk = mask.shape
    nqb = -(-Sq // block_q)
    nkb = -(-Sk // block_k)
    out = np.zeros((nqb, nkb), np.uint8)
    for a in range(nqb):
        for c in range(nkb):
            tile = mask[a * block_q:(a + 1) * block_q, c * block_k:(c + 1) * block_k]
            whole = tile.shape == (block_q, block_k)
            if not tile.any():
                out[a, c] = SKIP
            elif whole and tile.all():
                out[a, c] = FULL
            else:
                out[a, c] = PARTIAL
    return out


def ranges_from_status(status):
    """Per query block the inclusive [first, last] non-SKIP key block (first > last when
    none), and per key block the same over query blocks."""
    nqb, nkb = status.shape
    q_rng = np.zeros((nqb, 2), np.int32)
    k_rng = np.zeros((nkb, 2), np.int32)
    for a in range(nqb):
        nz = np.nonzero(status[a] != SKIP)[0]
        q_rng[a] = (nz[0], nz[-1]) if nz.size else (0, -1)
    for c in range(nkb):
        nz = np.nonzero(status[:, c] != SKIP)[0]
        k_rng[c] = (nz[0], nz[-1]) if nz.size else (0, -1)
    return q_rng, k_rng


def visible_pairs(seg_q, seg_k, q_offset=0, k_offset=0, causal=True) -> int:
    """Number of visible (query, key) pairs, by counting the mask."""
    return int(visibility(seg_q, seg_k, q_offset, k_offset, causal).sum())
