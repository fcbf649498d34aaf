"""GPU parity of the split-KV decode call (lwm_attn_decode): few query rows against a long
key/value cache.  Small cases are compared element by element with the float64 oracle and
with the ordinary forward on the same inputs; the 1M-token cache is checked on sampled
heads (every query row, each from its full masked score row) and through the Q = 0 closed
form on every row and head."""
import math

import numpy as np
import pytest

import lwm_inputs as li
from oracle import attention as A
from gpu_helpers import TOL_LSE, TOL_O, f64, host_f64, max_abs, say, seg_dev, to_dev
from test_gpu_small import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")

CASES = [
    # name, seed, B, H, Sq, Sk, layout, q_off (None: the cache's last Sq positions), causal, pad
    ("one_token", 11, 2, 3, 1, 5000, "single", None, True, False),
    ("rows16_packed", 12, 1, 2, 16, 70001, "packed", None, True, False),
    ("rows_over_waves", 13, 1, 2, 100, 3000, "packed", None, True, False),
    ("two_query_tiles", 14, 1, 1, 200, 40000, "single", None, True, False),
    ("cache_below_one_tile", 15, 1, 2, 4, 10, "single", None, True, False),
    ("noncausal_packed", 16, 1, 2, 8, 20000, "packed", 0, False, False),
    ("padding_rows", 17, 2, 2, 5, 9000, "packed", None, True, True),
    ("queries_before_cache_end", 18, 1, 2, 3, 6000, "single", 2500, True, False),
]


def decode(desc, q, k, v, sq, sk):
    table = lwm.lwm_attn_build_block_table(desc, sq, sk)
    ws = torch.empty(max(lwm.lwm_attn_decode_workspace_bytes(desc), 16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lwm.lwm_attn_decode(desc, q, k, v, sq, sk, table, o, lse, ws)
    return o, lse, table


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle_and_forward(case):
    name, seed, B, H, Sq, Sk, layout, q_off, causal, pad = case
    D = 128
    q_off = Sk - Sq if q_off is None else q_off
    say(f"decode case {name}: B={B} H={H} Sq={Sq} Sk={Sk} q_off={q_off} causal={causal}")
    x, seg_q, seg_k = make_case(seed, B, H, Sq, Sk, D, "bf16", layout, q_off, 0, pad)
    scale = 1 / math.sqrt(D)
    q, k, v = (host_f64(x[n], "bf16") for n in ("q", "k", "v"))
    o_ref, lse_ref = A.forward(q, k, v, seg_q, seg_k, scale, causal, q_off, 0)
    qd, kd, vd = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    desc = lwm.make_desc(B, H, Sq, Sk, D, torch.bfloat16, scale=scale, causal=causal,
                         q_offset=q_off)
    o, lse, table = decode(desc, qd, kd, vd, sq, sk)
    o_f = torch.empty_like(qd)
    lse_f = torch.empty_like(lse)
    lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, qd, kd, vd, sq, sk, table, o=o_f, lse=lse_f)
    torch.cuda.synchronize()
    eo, el = max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref)
    fo, fl = max_abs(f64(o), f64(o_f)), max_abs(f64(lse), f64(lse_f))
    say(f"  vs oracle: O {eo:.2e} LSE {el:.2e}; vs forward: O {fo:.2e} LSE {fl:.2e}")
    assert np.array_equal(np.isinf(f64(lse)), np.isinf(lse_ref))
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE
    assert fo <= TOL_O["bf16"] and fl <= TOL_LSE


def test_decode_empty_cache():
    """No keys at all: every row sees nothing, so O = 0 and LSE = -inf by definition."""
    say("decode: empty cache")
    B, H, Sq, D = 1, 2, 3, 128
    q = torch.ones((B, H, Sq, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((B, H, 0, D), dtype=torch.bfloat16, device="cuda")
    sq = torch.zeros((B, Sq), dtype=torch.int32, device="cuda")
    sk = torch.zeros((B, 0), dtype=torch.int32, device="cuda")
    desc = lwm.make_desc(B, H, Sq, 0, D, torch.bfloat16, q_offset=0)
    o, lse, _ = decode(desc, q, kv, kv, sq, sk)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_decode_workspace_reuse_across_shapes():
    """One workspace serves two calls of different sizes in a row; each call's result
    stands alone (nothing stale from the previous call leaks in)."""
    say("decode: workspace reuse")
    D = 128
    outs = []
    big = None
    for (seed, Sq, Sk) in ((21, 16, 30000), (22, 3, 5000)):
        x, seg_q, seg_k = make_case(seed, 1, 2, Sq, Sk, D, "bf16", "single", Sk - Sq, 0)
        qd, kd, vd = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
        sq, sk = seg_dev(seg_q), seg_dev(seg_k)
        desc = lwm.make_desc(1, 2, Sq, Sk, D, torch.bfloat16, q_offset=Sk - Sq)
        if big is None:
            big = torch.empty(lwm.lwm_attn_decode_workspace_bytes(desc), dtype=torch.uint8,
                              device="cuda")
        assert big.numel() >= lwm.lwm_attn_decode_workspace_bytes(desc)
        table = lwm.lwm_attn_build_block_table(desc, sq, sk)
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
        lwm.lwm_attn_decode(desc, qd, kd, vd, sq, sk, table, o, lse, big)
        q, k, v = (host_f64(x[n], "bf16") for n in ("q", "k", "v"))
        o_ref, lse_ref = A.forward(q, k, v, seg_q, seg_k, 1 / math.sqrt(D), True, Sk - Sq, 0)
        torch.cuda.synchronize()
        outs.append((max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref)))
    say(f"  {outs}")
    assert all(eo <= TOL_O["bf16"] and el <= TOL_LSE for eo, el in outs)


def decode_full(w):
    seg_q, seg_k = li.workload_segment_ids(w)
    q = li.device_normal((w.B, w.H, w.Sq, w.D), w.seed, w.value_scale, 0, torch.bfloat16, "cuda")
    k = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 1, torch.bfloat16, "cuda")
    v = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 2, torch.bfloat16, "cuda")
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    desc = lwm.make_desc(w.B, w.H, w.Sq, w.Sk, w.D, torch.bfloat16, q_offset=w.q_offset)
    return desc, q, k, v, sq, sk, seg_q, seg_k


@pytest.mark.parametrize("wname", ["decode_1m_q1", "decode_1m_q16"])
def test_decode_1m_cache(wname):
    w = li.WORKLOADS[wname]
    say(f"{w.name}: Sq={w.Sq} against a {w.Sk}-token cache; sampled heads, then Q = 0 on all rows")
    desc, q, k, v, sq, sk, seg_q, seg_k = decode_full(w)
    o, lse, table = decode(desc, q, k, v, sq, sk)
    torch.cuda.synchronize()
    heads = li.sample_rows(w, [w.Sk])
    rows = np.arange(w.Sq)
    worst = [0.0, 0.0]
    for h in heads:
        qh = q[0, h].float().cpu().numpy().astype(np.float64)
        kh = k[0, h].float().cpu().numpy().astype(np.float64)
        vh = v[0, h].float().cpu().numpy().astype(np.float64)
        o_ref, lse_ref = A.forward_rows(qh, kh, vh, seg_q[0], seg_k[0], w.q_offset + rows, w.scale)
        worst[0] = max(worst[0], max_abs(f64(o[0, h]), o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse[0, h]), lse_ref))
        del kh, vh
    say(f"  sampled heads {sorted(heads)}: max-abs O {worst[0]:.2e} LSE {worst[1]:.2e}")
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE
    # Q = 0: every visible key has score 0, so LSE_i = ln(count_i) and O_i is the mean of the
    # visible values; row i sees keys 0 .. q_offset + i
    qz = torch.zeros_like(q)
    o0, lse0, _ = decode(desc, qz, k, v, sq, sk)
    torch.cuda.synchronize()
    cnt = w.q_offset + rows + 1.0
    e_lse = max_abs(f64(lse0)[0], np.log(cnt)[None].repeat(w.H, 0))
    e_o = 0.0
    for h in (0, w.H - 1):
        vh = v[0, h].float().cpu().numpy().astype(np.float64)
        base = vh[: w.q_offset].sum(axis=0)
        ref = (base[None] + np.cumsum(vh[w.q_offset:w.q_offset + w.Sq], axis=0)) / cnt[:, None]
        e_o = max(e_o, max_abs(f64(o0[0, h]), ref))
        del vh
    say(f"  Q = 0: max-abs LSE {e_lse:.2e} (all rows, all heads), O {e_o:.2e} (2 heads)")
    assert e_lse <= TOL_LSE and e_o <= TOL_O["bf16"]


def test_plain_forward_on_1m_cache_walks_status_chunks():
    """The plain forward on the 16-row decode inputs: one query tile sees 16384 key tiles,
    staged in LDS 2048 at a time.  Against the decode result and, on two heads, the oracle."""
    w = li.WORKLOADS["decode_1m_q16"]
    say(f"{w.name}: plain forward over 16384 key tiles vs decode and the oracle")
    desc, q, k, v, sq, sk, seg_q, seg_k = decode_full(w)
    o_d, lse_d, table = decode(desc, q, k, v, sq, sk)
    o_f = torch.empty_like(q)
    lse_f = torch.empty_like(lse_d)
    lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, q, k, v, sq, sk, table, o=o_f, lse=lse_f)
    torch.cuda.synchronize()
    fo, fl = max_abs(f64(o_f), f64(o_d)), max_abs(f64(lse_f), f64(lse_d))
    rows = np.arange(w.Sq)
    worst = [0.0, 0.0]
    for h in (0, w.H - 1):
        qh = q[0, h].float().cpu().numpy().astype(np.float64)
        kh = k[0, h].float().cpu().numpy().astype(np.float64)
        vh = v[0, h].float().cpu().numpy().astype(np.float64)
        o_ref, lse_ref = A.forward_rows(qh, kh, vh, seg_q[0], seg_k[0], w.q_offset + rows, w.scale)
        worst[0] = max(worst[0], max_abs(f64(o_f[0, h]), o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse_f[0, h]), lse_ref))
        del kh, vh
    say(f"  forward vs decode: O {fo:.2e} LSE {fl:.2e}; vs oracle: O {worst[0]:.2e} LSE {worst[1]:.2e}")
    assert fo <= TOL_O["bf16"] and fl <= TOL_LSE
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE
