"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This module holds data only: workload shapes, segment layouts, seeded normal draws,
bf16 rounding of generated values and row sampling. It contains none of the attention
arithmetic, so the HIP path and the CPU oracle can both be fed from it without sharing
any computation.

Workload shapes follow the LWM pages (deep dive "LWM: million-token video-language world
model", sections "模型结构 / model structure" and "Masked sequence packing"): a LLaMA-2-7B
shaped attention (32 heads of width 128), text documents packed together with video
segments of 256 VQGAN codes plus one frame delimiter per frame.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np

TOKENS_PER_FRAME = 257  # 256 VQGAN codes + one <eof>/<eov> delimiter per frame


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload.

    Sq query rows sit at global positions q_offset .. q_offset+Sq-1; the Sk keys at
    k_offset .. k_offset+Sk-1.  For the ring share, Sk covers every KV chunk of the ring
    (n_chunks chunks of Sk // n_chunks keys each, chunk c at global offset c * chunk).
    """

    name: str
    B: int
    H: int
    D: int
    Sq: int
    Sk: int
    dtype: str  # "f32" or "bf16"
    seed: int
    layout: str  # "fixed3", "single", "packed"
    q_offset: int = 0
    n_chunks: int = 1
    backward: bool = False
    sample_heads: int = 0
    sample_rows_per_head: int = 0
    value_scale: float = 0.5
    grad_scale: float = 0.1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    "tiny_packed_f32": Workload("tiny_packed_f32", 1, 1, 64, 256, 256, "f32", 1, "fixed3",
                                value_scale=1.0, backward=True),
    "single_32k": Workload("single_32k", 1, 32, 128, 32768, 32768, "bf16", 2, "single",
                           sample_heads=8, sample_rows_per_head=64),
    "packed_64k": Workload("packed_64k", 1, 32, 128, 65536, 65536, "bf16", 3, "packed",
                           sample_heads=8, sample_rows_per_head=64),
    "ring_share_128k_x8": Workload("ring_share_128k_x8", 1, 32, 128, 131072, 8 * 131072, "bf16", 4,
                                   "single", q_offset=5 * 131072, n_chunks=8,
                                   sample_heads=4, sample_rows_per_head=64),
    "packed_128k_fwd_bwd": Workload("packed_128k_fwd_bwd", 1, 32, 128, 131072, 131072, "bf16", 5,
                                    "packed", backward=True, sample_heads=4,
                                    sample_rows_per_head=64),
    # decode: the newest tokens of one sequence against its 1M-token key/value cache (the
    # pages' 1M-token inference), one token per step and a block of 16 rows
    "decode_1m_q1": Workload("decode_1m_q1", 1, 32, 128, 1, 1 << 20, "bf16", 6, "single",
                             q_offset=(1 << 20) - 1, sample_heads=8, sample_rows_per_head=1),
    "decode_1m_q16": Workload("decode_1m_q16", 1, 32, 128, 16, 1 << 20, "bf16", 7, "single",
                              q_offset=(1 << 20) - 16, sample_heads=4, sample_rows_per_head=16),
}


# ----------------------------------------------------------------------------------------
# segment layouts
# ----------------------------------------------------------------------------------------

FIXED3_LENGTHS = (100, 90, 66)


def draw_packed_segments(total: int, seed: int) -> List[Tuple[str, int]]:
    """Draw (kind, length) segments until they fill `total` tokens.

    Kind is text or vision with probability 1/2 each.  Text lengths are log-uniform in
    [1024, 16384]; a vision segment holds n frames of 257 tokens with n uniform in 4..32.
    The last segment is cut so the lengths sum to exactly `total`.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out: List[Tuple[str, int]] = []
    filled = 0
    while filled < total:
        if rng.random() < 0.5:
            kind = "text"
            length = int(math.floor(math.exp(rng.uniform(math.log(1024), math.log(16384)))))
        else:
            kind = "vision"
            length = TOKENS_PER_FRAME * int(rng.integers(4, 33))
        length = min(length, total - filled)
        out.append((kind, length))
        filled += length
    return out


def segment_ids_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """Consecutive ids 0, 1, 2, ... repeated over each segment's tokens (int32)."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))


def workload_segments(w: Workload) -> List[Tuple[str, int]]:
    """Segment list covering the *global* token range 0 .. q_offset + Sq (or Sk) - 1."""
    total = max(w.q_offset + w.Sq, w.Sk)
    if w.layout == "fixed3":
        assert sum(FIXED3_LENGTHS) == total
        return [("text", n) for n in FIXED3_LENGTHS]
    if w.layout == "single":
        return [("text", total)]
    if w.layout == "packed":
        return draw_packed_segments(total, w.seed)
    raise ValueError(w.layout)


def workload_segment_ids(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """(seg_q [B,Sq], seg_k [B,Sk]) int32, identical across the batch."""
    ids = segment_ids_from_lengths([n for _, n in workload_segments(w)])
    seg_q = np.broadcast_to(ids[w.q_offset:w.q_offset + w.Sq], (w.B, w.Sq)).copy()
    seg_k = np.broadcast_to(ids[:w.Sk], (w.B, w.Sk)).copy()
    return seg_q, seg_k


def segment_bounds(lengths: Sequence[int]) -> List[Tuple[int, int]]:
    """[(start, end_exclusive)] per segment."""
    out, pos = [], 0
    for n in lengths:
        out.append((pos, pos + n))
        pos += n
    return out


# ----------------------------------------------------------------------------------------
# values
# ----------------------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def host_normal(shape, seed: int, scale: float, stream: int = 0) -> np.ndarray:
    """float32 N(0,1)*scale from PCG64(seed) jumped by `stream` (Q, K, V, dO use streams 0..3)."""
    bitgen = np.random.PCG64(seed)
    if stream:
        bitgen = bitgen.jumped(stream)
    rng = np.random.Generator(bitgen)
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def host_tensors(w: Workload, Sq: int | None = None, Sk: int | None = None, heads: int | None = None):
    """Host-generated Q, K, V, dO for a (possibly shrunk) workload.

    Returns a dict of arrays: float32 for dtype "f32"; uint16 bf16 bit patterns for "bf16".
    """
    Sq = w.Sq if Sq is None else Sq
    Sk = w.Sk if Sk is None else Sk
    H = w.H if heads is None else heads
    shapes = {"q": (w.B, H, Sq, w.D), "k": (w.B, H, Sk, w.D), "v": (w.B, H, Sk, w.D),
              "do": (w.B, H, Sq, w.D)}
    out = {}
    for i, name in enumerate(("q", "k", "v", "do")):
        sc = w.grad_scale if name == "do" else w.value_scale
        x = host_normal(shapes[name], w.seed, sc, stream=i)
        out[name] = x if w.dtype == "f32" else bf16_bits_from_f32(x)
    return out


def device_normal(shape, seed: int, scale: float, stream: int, dtype, device):
    """torch tensor N(0,1)*scale drawn on `device` from a seeded torch generator, cast to dtype
    (round to nearest even).  Used where host generation of GiB-sized inputs would be slow."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + stream)
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(generator=g)
    x.mul_(scale)
    return x.to(dtype)


# ----------------------------------------------------------------------------------------
# row sampling
# ----------------------------------------------------------------------------------------

def forced_rows(Sq: int, q_offset: int, lengths: Sequence[int]) -> List[int]:
    """Local query rows that every sampled head checks: the ends of the query range, the
    first and last row of every segment that meets it, and the rows around 64 and 128."""
    rows = {0, Sq - 1, 63, 64, 127, 128}
    for s, e in segment_bounds(lengths):
        for g in (s, e - 1):
            if q_offset <= g < q_offset + Sq:
                rows.add(g - q_offset)
    return sorted(r for r in rows if 0 <= r < Sq)


def sample_rows(w: Workload, lengths: Sequence[int], seed_offset: int = 0):
    """Seeded (head, local row) samples: a fixed head subset, per head the forced rows plus
    uniform draws without replacement up to `sample_rows_per_head` rows."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 7919 + seed_offset))
    heads = np.sort(rng.choice(w.H, size=w.sample_heads, replace=False))
    forced = forced_rows(w.Sq, w.q_offset, lengths)
    out = {}
    for h in heads:
        rows = set(forced[: w.sample_rows_per_head])
        while len(rows) < w.sample_rows_per_head:
            rows.add(int(rng.integers(0, w.Sq)))
        out[int(h)] = np.array(sorted(rows), dtype=np.int64)
    return out

