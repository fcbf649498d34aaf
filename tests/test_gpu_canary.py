"""Race canary: the bf16 kernels built with a wait for the wave's loads and a workgroup
barrier after every phase of a tile step (liblwm_attn_canary.so) must give results identical
bit for bit to the normal build, whose schedule relies on one barrier per tile.  A race in
the normal schedule (a load into a buffer another wave still reads, a read of a tile before
its loads landed) would show as a difference."""
import numpy as np
import pytest

import lwm_inputs as li
from gpu_helpers import say, seg_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def everything(q, k, v, do, sq, sk, q_off=0, k_off=0):
    """Forward (FINAL and PARTIAL), backward and split-KV decode outputs."""
    o, lse, table = lwm.attention_forward(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, sq, sk, table, q_offset=q_off,
                                        k_offset=k_off)
    m, l, acc = lwm.attention_partial(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off, table=table)
    od, lsed, _ = lwm.attention_decode(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off, table=table)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv, "m": m, "l": l, "acc": acc,
            "O_decode": od, "LSE_decode": lsed}


CASES = [
    # name, B, H, S, layout, seed
    ("packed_ragged", 1, 2, 1000, "packed", 61),
    ("packed_padding_b2", 2, 2, 1500, "padded", 62),
    ("single_147456_two_status_chunks", 1, 2, 147456, "single", 63),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_canary_build_is_bit_identical(case):
    name, B, H, S, layout, seed = case
    say(f"race canary {name}: B={B} H={H} S={S}")
    rng = np.random.default_rng(seed)
    if layout == "single":
        ids = np.zeros((B, S), np.int32)
    else:
        rows = []
        for _ in range(B):
            lengths = [n for _, n in li.draw_packed_segments(S, int(rng.integers(0, 1 << 20)))]
            r = li.segment_ids_from_lengths(lengths).astype(np.int32)
            if layout == "padded":
                r[rng.random(S) < 0.1] = -1
            rows.append(r)
        ids = np.stack(rows)
    sq = seg_dev(ids)
    q, k, v, do = (li.device_normal((B, H, S, 128), seed, 0.1 if i == 3 else 0.5, i, torch.bfloat16,
                                    "cuda") for i in range(4))
    normal = everything(q, k, v, do, sq, sq)
    with lwm.active_library(lwm.CANARY_LIB_PATH):
        canary = everything(q, k, v, do, sq, sq)
    diff = {n: bool(torch.equal(normal[n], canary[n])) for n in normal}
    say("  identical: " + ", ".join(f"{n} {d}" for n, d in diff.items()))
    assert all(diff.values()), diff
