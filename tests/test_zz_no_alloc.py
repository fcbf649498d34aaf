"""lwm_attn_decode_noalloc (slice states in the library's static device buffer) against
lwm_attn_decode (slice states in a caller workspace) through the C-ABI, on two calls in a
row, the second with a smaller input, and both against the float64 oracle."""
import math

import numpy as np
import pytest

import lwm_inputs as li
from oracle import attention as A
from gpu_helpers import TOL_LSE, TOL_O, f64, max_abs, say, seg_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def decode_both(q, k, v, seg_q, seg_k, q_offset):
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    desc = lwm.make_desc(B, H, Sq, Sk, D, torch.bfloat16, q_offset=q_offset)
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    table = lwm.lwm_attn_build_block_table(desc, sq, sk)
    ws_bytes = lwm.lwm_attn_decode_workspace_bytes(desc)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    o_ws, lse_ws = torch.empty_like(q), torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    lwm.lwm_attn_decode(desc, q, k, v, sq, sk, table, o_ws, lse_ws, ws)
    o_st = torch.full_like(q, float("nan"))
    lse_st = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    lwm.lwm_attn_decode_noalloc(desc, q, k, v, sq, sk, table, o_st, lse_st)
    torch.cuda.synchronize()
    return ws_bytes, (o_ws, lse_ws), (o_st, lse_st)


def test_decode_noalloc_matches_workspace_decode_twice():
    # call 1: 128 new rows per head against a 262144-token cache.  The default split would
    # need more slice states than the static buffer holds, so the call uses fewer, longer
    # slices
    B, H, Sq, Sk, D, seed = 1, 32, 128, 262144, 128, 91
    say(f"no-alloc decode call 1: B={B} H={H} Sq={Sq} Sk={Sk}")
    q, k, v = (li.device_normal((B, H, S, D), seed, 0.5, i, torch.bfloat16, "cuda")
               for i, S in enumerate((Sq, Sk, Sk)))
    seg_q = np.zeros((B, Sq), np.int32)
    seg_k = np.zeros((B, Sk), np.int32)
    q_off = Sk - Sq
    ws_bytes, (o_ws, lse_ws), (o_st, lse_st) = decode_both(q, k, v, seg_q, seg_k, q_off)
    assert ws_bytes > lwm.DECODE_SCRATCH_BYTES
    e_o, e_l = max_abs(f64(o_st), f64(o_ws)), max_abs(f64(lse_st), f64(lse_ws))
    say(f"  static vs workspace: O {e_o:.2e} LSE {e_l:.2e}")
    assert e_o <= TOL_O["bf16"] and e_l <= TOL_LSE
    assert not torch.isnan(o_st).any() and not torch.isnan(lse_st).any()
    rows = np.array([0, 1, 63, 64, 126, 127])
    worst = [0.0, 0.0]
    for h in (0, 17, 31):
        kh, vh = (t[0, h].float().cpu().numpy().astype(np.float64) for t in (k, v))
        qh = q[0, h].float().cpu().numpy().astype(np.float64)[rows]
        o_ref, lse_ref = A.forward_rows(qh, kh, vh, seg_q[0][rows], seg_k[0], q_off + rows,
                                        1 / math.sqrt(D))
        worst[0] = max(worst[0], max_abs(f64(o_st[0, h])[rows], o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse_st[0, h])[rows], lse_ref))
    say(f"  static vs oracle on sampled rows: O {worst[0]:.2e} LSE {worst[1]:.2e}")
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE
    del q, k, v, o_ws, lse_ws, o_st, lse_st

    # call 2, smaller: two batch rows of packed samples with padding, 16 new rows per head;
    # the buffer still holds call 1's states, which must not leak into this result
    B, H, Sq, Sk = 2, 4, 16, 5000
    say(f"no-alloc decode call 2: B={B} H={H} Sq={Sq} Sk={Sk} packed with padding")
    rng = np.random.default_rng(92)
    ids = []
    for _ in range(B):
        lengths = [n for _, n in li.draw_packed_segments(Sk, int(rng.integers(0, 1000)))]
        lid = li.segment_ids_from_lengths(lengths).astype(np.int32)
        lid[rng.random(Sk) < 0.05] = -1
        ids.append(lid)
    seg_k = np.stack(ids)
    seg_q = seg_k[:, Sk - Sq:].copy()
    x = {n: li.bf16_bits_from_f32(li.host_normal((B, H, S, D), 93, 0.5, i))
         for i, (n, S) in enumerate((("q", Sq), ("k", Sk), ("v", Sk)))}
    dev = {n: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for n, b in x.items()}
    ws_bytes2, (o_ws, lse_ws), (o_st, lse_st) = decode_both(dev["q"], dev["k"], dev["v"], seg_q,
                                                            seg_k, Sk - Sq)
    assert ws_bytes2 < ws_bytes
    f = {n: li.bf16_bits_to_f64(b) for n, b in x.items()}
    o_ref, lse_ref = A.forward(f["q"], f["k"], f["v"], seg_q, seg_k, 1 / math.sqrt(D), True,
                               Sk - Sq, 0)
    e = [max_abs(f64(o_st), f64(o_ws)), max_abs(f64(lse_st), f64(lse_ws)),
         max_abs(f64(o_st), o_ref), max_abs(f64(lse_st), lse_ref)]
    say("  static vs workspace: O {:.2e} LSE {:.2e}; static vs oracle: O {:.2e} LSE {:.2e}".format(*e))
    assert np.array_equal(np.isinf(f64(lse_st)), np.isinf(lse_ref))
    assert e[0] <= TOL_O["bf16"] and e[1] <= TOL_LSE
    assert e[2] <= TOL_O["bf16"] and e[3] <= TOL_LSE
