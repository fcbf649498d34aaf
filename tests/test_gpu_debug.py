"""Device checks: liblwm_attn_debug.so is the library built with LWM_DEBUG, in which every
kernel checks the indices it derives from the block table (query and key ranges, tile
statuses, status-chunk slots) and its launch shape against the extents they index, and the
merge checks that an empty state carries l = 0.  A failed check is recorded on the device
rather than trapping.  On valid inputs no check may fail and the checks must not change a
single output bit; the self test shows that a failed check is reported and then cleared."""
import numpy as np
import pytest

import lwm_inputs as li
from gpu_helpers import say, seg_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def test_self_test_is_reported_and_cleared():
    with lwm.active_library(lwm.DEBUG_LIB_PATH):
        assert lwm.lwm_attn_debug_status()[0] == 0  # clear anything earlier
        rc, w0, w1 = lwm.lwm_attn_debug_status(self_test=True)
        say(f"self test: rc {rc} words {w0:#x} {w1:#x}")
        assert rc == 0 and w0 == 1 << 31 and w1 >> 24 == 31
        assert lwm.lwm_attn_debug_status() == (0, 0, 0)


def everything(q, k, v, do, sq, sk, q_off=0, k_off=0, causal=True):
    """Table, forward (FINAL and PARTIAL), backward and, for bf16, split-KV decode."""
    o, lse, table = lwm.attention_forward(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off,
                                          causal=causal)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, sq, sk, table, q_offset=q_off,
                                        k_offset=k_off, causal=causal)
    m, l, acc = lwm.attention_partial(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off,
                                      causal=causal, table=table)
    out = {"table": table, "O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv, "m": m, "l": l,
           "acc": acc}
    if q.dtype == torch.bfloat16:
        od, lsed, _ = lwm.attention_decode(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off,
                                           causal=causal, table=table)
        out.update({"O_decode": od, "LSE_decode": lsed})
    torch.cuda.synchronize()
    return out


def table_bytes(table, B, Sq, Sk):
    """The parts of a block table that the builder writes (ranges, statuses, block statistics;
    64-row blocks, each part on a 256-byte boundary), without the padding between them."""
    raw = table.cpu().numpy()
    nqb, nkb = -(-Sq // 64), -(-Sk // 64)
    al = lambda x: (x + 255) // 256 * 256
    sizes = [B * nqb * 8, B * nkb * 8, B * nqb * nkb, B * nqb * 16, B * nkb * 16]
    parts, off = [], 0
    for n in sizes:
        parts.append(raw[off:off + n])
        off += al(n)
    return np.concatenate(parts)


def layout_ids(B, S, layout, rng):
    if layout == "single":
        return np.zeros((B, S), np.int32)
    rows = []
    for _ in range(B):
        lengths = [n for _, n in li.draw_packed_segments(S, int(rng.integers(0, 1 << 20)))]
        r = li.segment_ids_from_lengths(lengths).astype(np.int32)
        if layout == "padded":
            r[rng.random(S) < 0.1] = -1
        rows.append(r)
    return np.stack(rows)


CASES = [
    # name, B, H, Sq, Sk, D, dtype, layout, q_offset, k_offset, causal, seed
    ("bf16_packed_ragged", 1, 2, 1000, 1000, 128, "bf16", "packed", 0, 0, True, 71),
    ("bf16_padded_b2", 2, 2, 1500, 1500, 128, "bf16", "padded", 0, 0, True, 72),
    ("bf16_single_147456_two_status_chunks", 1, 2, 147456, 147456, 128, "bf16", "single", 0, 0,
     True, 73),
    ("bf16_offsets_sq_ne_sk", 1, 2, 700, 1300, 128, "bf16", "single", 1200, 0, True, 74),
    ("bf16_noncausal_packed", 1, 2, 900, 900, 128, "bf16", "packed", 0, 0, False, 75),
    ("f32_packed_ragged", 1, 2, 300, 300, 64, "f32", "packed", 0, 0, True, 76),
    ("f32_offsets_d32", 2, 1, 200, 333, 32, "f32", "padded", 133, 0, True, 77),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_debug_build_checks_pass_and_change_nothing(case):
    name, B, H, Sq, Sk, D, dt, layout, q_off, k_off, causal, seed = case
    say(f"debug build {name}: B={B} H={H} Sq={Sq} Sk={Sk} D={D} {dt}")
    rng = np.random.default_rng(seed)
    ids_q = layout_ids(B, Sq, layout, rng)
    ids_k = ids_q if Sk == Sq else layout_ids(B, Sk, layout, rng)
    sq, sk = seg_dev(ids_q), seg_dev(ids_k)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q, do = (li.device_normal((B, H, Sq, D), seed, s, i, tdt, "cuda") for i, s in ((0, 0.5), (3, 0.1)))
    k, v = (li.device_normal((B, H, Sk, D), seed, 0.5, i, tdt, "cuda") for i in (1, 2))
    normal = everything(q, k, v, do, sq, sk, q_off, k_off, causal)
    with lwm.active_library(lwm.DEBUG_LIB_PATH):
        assert lwm.lwm_attn_debug_status()[0] == 0
        checked = everything(q, k, v, do, sq, sk, q_off, k_off, causal)
        rc, w0, w1 = lwm.lwm_attn_debug_status()
    say(f"  failed checks {w0:#x} (first {w1:#x})")
    assert rc == 0 and w0 == 0 and w1 == 0
    diff = {n: bool(torch.equal(normal[n], checked[n])) for n in normal if n != "table"}
    diff["table"] = bool(np.array_equal(table_bytes(normal["table"], B, Sq, Sk),
                                        table_bytes(checked["table"], B, Sq, Sk)))
    say("  identical: " + ", ".join(f"{n} {d}" for n, d in diff.items()))
    assert all(diff.values()), diff


def test_debug_build_ring_share_merges():
    """The ring share (partial forwards merged in ring order, finalised) through the debug
    build: the merge's state checks pass and the result is bit-identical."""
    B, H, S, D, n = 1, 2, 512, 128, 4
    say(f"debug build ring share: {n} chunks of {S}")
    q = li.device_normal((B, H, S, D), 78, 0.5, 0, torch.bfloat16, "cuda")
    ks = [li.device_normal((B, H, S, D), 78, 0.5, 1 + c, torch.bfloat16, "cuda") for c in range(n)]
    vs = [li.device_normal((B, H, S, D), 78, 0.5, 9 + c, torch.bfloat16, "cuda") for c in range(n)]
    seg = seg_dev(np.zeros((B, S), np.int32))
    args = dict(q_offset=(n - 1) * S, chunk_offsets=[c * S for c in range(n)],
                order=lwm.ring_order(n - 1, n))
    o1, l1, _ = lwm.ring_share_forward(q, ks, vs, seg, [seg] * n, **args)
    torch.cuda.synchronize()
    with lwm.active_library(lwm.DEBUG_LIB_PATH):
        assert lwm.lwm_attn_debug_status()[0] == 0
        o2, l2, _ = lwm.ring_share_forward(q, ks, vs, seg, [seg] * n, **args)
        rc, w0, w1 = lwm.lwm_attn_debug_status()
    say(f"  failed checks {w0:#x} (first {w1:#x})")
    assert rc == 0 and w0 == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
