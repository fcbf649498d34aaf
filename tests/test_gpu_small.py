"""GPU parity at sizes the float64 oracle finishes in seconds: every element of O, LSE,
partial states and gradients compared with the oracle on the same seeded inputs, across
several tiles, ragged tails, packed layouts, padding, offsets and the degenerate cases."""
import math

import numpy as np
import pytest

import lwm_inputs as li
from oracle import attention as A
from oracle import table as otab
import test_oracle_pins as pins
from gpu_helpers import (TOL_GRAD, TOL_LSE, TOL_O, check_grad, f64, host_f64, max_abs, say,
                         seg_dev, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def make_case(seed, B, H, Sq, Sk, D, dtype, layout="packed", q_off=0, k_off=0, pad=False,
              value_scale=0.5):
    rng = np.random.default_rng(seed)
    total = max(q_off + Sq, k_off + Sk)
    if layout == "single":
        ids = np.zeros(total, np.int32)
    elif layout == "packed":
        ids = pins.random_layout(rng, total, allow_padding=pad)
    elif layout == "tiny_segments":
        # many samples of one token (a row that sees only itself) among short ones, some of
        # them crossing tile edges
        pattern = [1, 1, 3, 1, 2, 1, 1, 63, 1, 1, 65, 1, 1, 1, 5, 130]
        lengths = (pattern * (total // sum(pattern) + 1))
        ids = li.segment_ids_from_lengths(lengths).astype(np.int32)[:total]
    elif layout.startswith("alternating"):
        # ids 0, 1, 0, 1, ... in runs of `run` tokens: a sample's tokens are not contiguous, so
        # SKIP tiles sit between live tiles of a row's (and a column's) range
        run = int(layout.split("_")[1])
        ids = ((np.arange(total) // run) % 2).astype(np.int32)
    else:
        raise ValueError(layout)
    seg_q = np.stack([ids[q_off:q_off + Sq]] * B)
    seg_k = np.stack([ids[k_off:k_off + Sk]] * B)
    x = {}
    for i, (name, S) in enumerate((("q", Sq), ("k", Sk), ("v", Sk), ("do", Sq))):
        sc = 0.1 if name == "do" else value_scale
        a = li.host_normal((B, H, S, D), seed, sc, stream=i)
        x[name] = a if dtype == "f32" else li.bf16_bits_from_f32(a)
    return x, seg_q, seg_k


def run_oracle(x, seg_q, seg_k, dtype, scale, causal, q_off, k_off, grads=True):
    q, k, v, do = (host_f64(x[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = A.forward(q, k, v, seg_q, seg_k, scale, causal, q_off, k_off)
    g = A.backward(q, k, v, do, seg_q, seg_k, scale, causal, q_off, k_off) if grads else None
    return o, lse, g


CASES = [
    # name, seed, B, H, Sq, Sk, layout, q_off, k_off, causal, pad
    ("single_ragged", 1, 1, 2, 700, 700, "single", 0, 0, True, False),
    ("packed_ragged", 2, 1, 2, 1000, 1000, "packed", 0, 0, True, False),
    ("packed_padding", 3, 2, 2, 640, 640, "packed", 0, 0, True, True),
    ("noncausal_packed", 4, 1, 2, 500, 500, "packed", 0, 0, False, False),
    ("offset_chunk", 5, 1, 2, 384, 448, "single", 896, 512, True, False),
    ("offset_diag", 6, 1, 1, 256, 256, "single", 768, 768, True, False),
    ("short_q", 7, 1, 3, 37, 300, "packed", 263, 0, True, False),
    ("one_row", 8, 1, 1, 1, 1, "single", 0, 0, True, False),
    ("few_keys", 9, 1, 2, 130, 3, "single", 0, 0, False, False),
    ("alternating_tiles", 10, 1, 2, 1024, 1024, "alternating_128", 0, 0, True, False),
    ("alternating_ragged", 11, 1, 2, 900, 900, "alternating_100", 0, 0, True, False),
    ("lone_segments", 12, 1, 2, 777, 777, "tiny_segments", 0, 0, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_forward_and_backward(case):
    name, seed, B, H, Sq, Sk, layout, q_off, k_off, causal, pad = case
    D = 128
    say(f"bf16 case {name}: B={B} H={H} Sq={Sq} Sk={Sk} offs={q_off},{k_off} causal={causal}")
    x, seg_q, seg_k = make_case(seed, B, H, Sq, Sk, D, "bf16", layout, q_off, k_off, pad)
    if layout.startswith("alternating"):
        # the layout does what it is for: SKIP tiles between live tiles of a row and a column
        st = otab.classify(seg_q[0], seg_k[0], 64, 64, q_off, k_off, causal)
        def gap(v):
            live = np.nonzero(v != otab.SKIP)[0]
            return live.size > 1 and np.any(v[live[0]:live[-1] + 1] == otab.SKIP)
        assert any(gap(r) for r in st) and any(gap(c) for c in st.T)
    scale = 1 / math.sqrt(D)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = run_oracle(x, seg_q, seg_k, "bf16", scale, causal,
                                                          q_off, k_off)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o, lse, table = lwm.attention_forward(q, k, v, sq, sk, causal=causal, q_offset=q_off,
                                          k_offset=k_off)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, sq, sk, table, causal=causal,
                                        q_offset=q_off, k_offset=k_off)
    torch.cuda.synchronize()
    eo, el = max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref)
    say(f"  max-abs O {eo:.2e} LSE {el:.2e}")
    assert np.array_equal(np.isinf(f64(lse)), np.isinf(lse_ref))
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE
    for n, g, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        check_grad(n, f64(g), r, "bf16")
    if layout == "tiny_segments":
        # a one-token sample attends to itself alone: O_i = v_i, dQ_i = 0 and, no other row
        # seeing its key, dV_i = dO_i and dK_i = 0
        ids = seg_q[0]
        lone = np.nonzero((np.r_[True, ids[1:] != ids[:-1]]) & (np.r_[ids[:-1] != ids[1:], True]))[0]
        # (up to the bf16 rounding of O, which leaves dP - Delta = <dO, v - O> a few 1e-4)
        say(f"  {lone.size} one-token samples")
        assert lone.size >= 25
        vv, dd = host_f64(x["v"], "bf16")[:, :, lone], host_f64(x["do"], "bf16")[:, :, lone]
        assert np.all(np.abs(f64(o)[:, :, lone] - vv) <= 2.0 ** -8 * np.abs(vv))
        assert np.all(np.abs(f64(dv)[:, :, lone] - dd) <= 2.0 ** -8 * np.abs(dd))
        assert np.abs(f64(dq)[:, :, lone]).max() <= 1e-4 and np.abs(f64(dk)[:, :, lone]).max() <= 1e-4


def test_tiny_packed_f32_forward_backward_partial():
    """The tiny packed fp32 workload: 256 tokens from segments 100/90/66, D = 64."""
    w = li.WORKLOADS["tiny_packed_f32"]
    t = li.host_tensors(w)
    seg_q, seg_k = li.workload_segment_ids(w)
    say("tiny packed f32")
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = run_oracle(t, seg_q, seg_k, "f32", w.scale, True, 0, 0)
    q, k, v, do = (to_dev(t[n], "f32") for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o, lse, table = lwm.attention_forward(q, k, v, sq, sk)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, sq, sk, table)
    m, l, acc = lwm.attention_partial(q, k, v, sq, sk, table=table)
    torch.cuda.synchronize()
    assert max_abs(f64(o), o_ref) <= TOL_O["f32"]
    assert max_abs(f64(lse), lse_ref) <= 1e-5
    for n, g, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        check_grad(n, f64(g), r, "f32")
    # partial state is (m, l, acc) relative to its own m: acc / l = O and m + ln l = LSE
    mm, ll, aa = f64(m), f64(l), f64(acc)
    assert max_abs(aa / ll[..., None], o_ref) <= TOL_O["f32"]
    assert max_abs(mm + np.log(ll), lse_ref) <= 1e-5


def test_f32_padding_offsets_ragged():
    say("f32 padding/offsets/ragged")
    x, seg_q, seg_k = make_case(21, 2, 2, 333, 200, 32, "f32", "packed", 150, 40, pad=True,
                                value_scale=1.0)
    scale = 1 / math.sqrt(32)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = run_oracle(x, seg_q, seg_k, "f32", scale, True, 150, 40)
    q, k, v, do = (to_dev(x[n], "f32") for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o, lse, table = lwm.attention_forward(q, k, v, sq, sk, q_offset=150, k_offset=40)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, sq, sk, table, q_offset=150, k_offset=40)
    torch.cuda.synchronize()
    assert max_abs(f64(o), o_ref) <= TOL_O["f32"]
    assert max_abs(f64(lse), lse_ref) <= 1e-5
    assert np.array_equal(np.isinf(f64(lse)), np.isinf(lse_ref))
    for n, g, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        check_grad(n, f64(g), r, "f32")


def test_bf16_partial_state():
    say("bf16 partial state")
    x, seg_q, seg_k = make_case(31, 1, 2, 300, 520, 128, "bf16", "single", 600, 128)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    m, l, acc = lwm.attention_partial(q, k, v, seg_dev(seg_q), seg_dev(seg_k), q_offset=600,
                                      k_offset=128)
    torch.cuda.synchronize()
    qf, kf, vf = (host_f64(x[n], "bf16") for n in ("q", "k", "v"))
    mask = A.visibility(seg_q[0], seg_k[0], 600, 128, True)
    for h in range(2):
        mo, lo, ao = A.partial_state(qf[0, h], kf[0, h], vf[0, h], mask, 1 / math.sqrt(128))
        o_ref, lse_ref = A.finalize_state((mo, lo, ao))
        mm, ll, aa = f64(m)[0, h], f64(l)[0, h], f64(acc)[0, h]
        assert max_abs(aa / ll[:, None], o_ref) <= TOL_O["bf16"]
        assert max_abs(mm + np.log(ll), lse_ref) <= TOL_LSE


def test_no_keys_gives_empty_rows():
    say("no keys")
    for dt, D in (("bf16", 128), ("f32", 64)):
        x, seg_q, seg_k = make_case(41, 1, 2, 100, 0, D, dt, "single")
        q = to_dev(x["q"], dt)
        k = to_dev(x["k"], dt)
        o, lse, _ = lwm.attention_forward(q, k, k, seg_dev(seg_q), seg_dev(seg_k))
        m, l, acc = lwm.attention_partial(q, k, k, seg_dev(seg_q), seg_dev(seg_k))
        torch.cuda.synchronize()
        assert np.all(f64(o) == 0) and np.all(f64(lse) == -np.inf)
        assert np.all(f64(m) == -np.inf) and np.all(f64(l) == 0) and np.all(f64(acc) == 0)


def test_all_padding_rows_are_empty():
    say("all padding")
    x, _, _ = make_case(42, 1, 1, 200, 200, 128, "bf16", "single")
    seg = -np.ones((1, 200), np.int32)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o, lse, _ = lwm.attention_forward(q, k, v, seg_dev(seg), seg_dev(seg))
    torch.cuda.synchronize()
    assert np.all(f64(o) == 0) and np.all(f64(lse) == -np.inf)


def test_forward_is_deterministic():
    say("determinism")
    x, seg_q, seg_k = make_case(51, 1, 4, 1500, 1500, 128, "bf16", "packed")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o1, l1, t = lwm.attention_forward(q, k, v, sq, sk)
    o2, l2, _ = lwm.attention_forward(q, k, v, sq, sk, table=t)
    g1 = lwm.attention_backward(q, k, v, o1, do, l1, sq, sk, t)
    g2 = lwm.attention_backward(q, k, v, o1, do, l1, sq, sk, t)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def random_state(rng, rows, D, empty_frac):
    m = rng.standard_normal(rows) * 3
    l = rng.uniform(0.5, 40, rows)
    acc = rng.standard_normal((rows, D)) * l[:, None]
    empty = rng.random(rows) < empty_frac
    m[empty] = -np.inf
    l[empty] = 0
    acc[empty] = 0
    return m.astype(np.float32), l.astype(np.float32), acc.astype(np.float32)


@pytest.mark.parametrize("D", [128, 64])
def test_merge_chunk(D):
    say(f"merge D={D}")
    rng = np.random.default_rng(61)
    rows = 3000
    s1 = random_state(rng, rows, D, 0.2)
    s2 = random_state(rng, rows, D, 0.2)
    ref = A.merge_states(*[tuple(np.asarray(a, np.float64) for a in s) for s in (s1, s2)])
    o_ref, lse_ref = A.finalize_state(ref)
    dev = lambda s: tuple(torch.from_numpy(a).cuda() for a in s)
    m, l, acc = dev(s1)
    mc, lc, accc = dev(s2)
    # finalize without write-back, into bf16 and fp32
    o16 = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((rows, D), dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    lwm.lwm_attn_merge_chunk(rows, D, m, l, acc, mc, lc, accc, finalize=True,
                             out_dtype=lwm.LWM_BF16, o=o16, lse=lse)
    lwm.lwm_attn_merge_chunk(rows, D, m, l, acc, mc, lc, accc, finalize=True,
                             out_dtype=lwm.LWM_F32, o=o32, lse=lse)
    torch.cuda.synchronize()
    assert np.array_equal(f64(m), np.asarray(s1[0], np.float64))  # untouched by finalize
    assert max_abs(f64(o32), o_ref) <= 1e-5 * max(1.0, np.abs(o_ref).max())
    assert max_abs(f64(o16), o_ref) <= 1e-2 * max(1.0, np.abs(o_ref).max())
    assert max_abs(f64(lse), lse_ref) <= 1e-5 * max(1.0, np.abs(lse_ref[np.isfinite(lse_ref)]).max())
    # merge with write-back, then finalize the running state alone
    lwm.lwm_attn_merge_chunk(rows, D, m, l, acc, mc, lc, accc, finalize=False)
    lwm.lwm_attn_merge_chunk(rows, D, m, l, acc, finalize=True, out_dtype=lwm.LWM_F32, o=o32, lse=lse)
    torch.cuda.synchronize()
    mm = f64(m)
    assert np.array_equal(np.isinf(mm), np.isinf(ref[0]))
    assert max_abs(f64(o32), o_ref) <= 1e-5 * max(1.0, np.abs(o_ref).max())


def test_ring_share_small():
    """8 KV chunks of 256 keys, query chunk at global offset 5 * 256, merged in ring order
    5, 4, 3, 2, 1, 0 (7 and 6 skipped), against one-shot attention over all keys."""
    chunk, N, H, D = 256, 8, 2, 128
    say("ring share small")
    rng_seed = 71
    x, seg_q, seg_all = make_case(rng_seed, 1, H, chunk, N * chunk, D, "bf16", "single",
                                  5 * chunk, 0)
    q = to_dev(x["q"], "bf16")
    k_all, v_all = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    ks = [k_all[:, :, c * chunk:(c + 1) * chunk].contiguous() for c in range(N)]
    vs = [v_all[:, :, c * chunk:(c + 1) * chunk].contiguous() for c in range(N)]
    segs = [seg_dev(seg_all[:, c * chunk:(c + 1) * chunk]) for c in range(N)]
    order = lwm.ring_order(5, N)
    assert order == [5, 4, 3, 2, 1, 0, 7, 6]
    o, lse, tables = lwm.ring_share_forward(q, ks, vs, seg_dev(seg_q), segs, q_offset=5 * chunk,
                                            chunk_offsets=[c * chunk for c in range(N)],
                                            order=order)
    torch.cuda.synchronize()
    assert sorted(tables) == [0, 1, 2, 3, 4, 5]
    o_ref, lse_ref, _ = run_oracle(x, seg_q, seg_all, "bf16", 1 / math.sqrt(D), True, 5 * chunk, 0,
                                   grads=False)
    assert max_abs(f64(o), o_ref) <= TOL_O["bf16"]
    assert max_abs(f64(lse), lse_ref) <= TOL_LSE
    # a different order gives the same result within the same bar
    o2, lse2, _ = lwm.ring_share_forward(q, ks, vs, seg_dev(seg_q), segs, q_offset=5 * chunk,
                                         chunk_offsets=[c * chunk for c in range(N)],
                                         order=[0, 3, 7, 1, 5, 2, 6, 4], tables=tables)
    torch.cuda.synchronize()
    assert max_abs(f64(o2), o_ref) <= TOL_O["bf16"]
    assert max_abs(f64(lse2), lse_ref) <= TOL_LSE


def test_q_zero_closed_form_all_rows():
    """Q = 0: every visible key weighs the same, so O is the mean of V over the row's
    visible keys (its segment up to itself) and LSE = ln(count), on every row and head."""
    say("q=0 closed form 8192 packed")
    S, H, D = 8192, 4, 128
    rng = np.random.default_rng(81)
    lengths = [n for _, n in li.draw_packed_segments(S, 81)]
    ids = li.segment_ids_from_lengths(lengths)[None]
    v_bits = li.bf16_bits_from_f32(li.host_normal((1, H, S, D), 81, 0.5, 2))
    k_bits = li.bf16_bits_from_f32(li.host_normal((1, H, S, D), 81, 0.5, 1))
    q = torch.zeros((1, H, S, D), dtype=torch.bfloat16, device="cuda")
    o, lse, _ = lwm.attention_forward(q, to_dev(k_bits, "bf16"), to_dev(v_bits, "bf16"),
                                      seg_dev(ids), seg_dev(ids))
    torch.cuda.synchronize()
    vf = li.bf16_bits_to_f64(v_bits)[0]
    ref = np.zeros_like(vf)
    cnt = np.zeros(S)
    for s, e in li.segment_bounds(lengths):
        cs = np.cumsum(vf[:, s:e], axis=1)
        n = np.arange(1, e - s + 1)
        ref[:, s:e] = cs / n[None, :, None]
        cnt[s:e] = n
    assert max_abs(f64(o)[0], ref) <= TOL_O["bf16"]
    assert max_abs(f64(lse)[0], np.log(cnt)[None].repeat(H, 0)) <= TOL_LSE


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_batch_rows_with_different_layouts(dt):
    """Each batch row has its own packing (segment cuts, padding, one row a single segment), so
    segment ids, the block table and the kernels must index the batch row correctly; forward,
    backward and decode against the oracle on every element."""
    B, H, Sq, Sk, q_off, k_off = 3, 2, 450, 520, 70, 0
    D = 128 if dt == "bf16" else 64
    say(f"batch rows with different layouts ({dt}): B={B} Sq={Sq} Sk={Sk} q_off={q_off}")
    rng = np.random.default_rng(77)
    total = max(q_off + Sq, k_off + Sk)
    layouts = [pins.random_layout(rng, total, allow_padding=False),
               pins.random_layout(rng, total, allow_padding=True),
               np.zeros(total, np.int32)]
    seg_q = np.stack([l[q_off:q_off + Sq] for l in layouts]).astype(np.int32)
    seg_k = np.stack([l[k_off:k_off + Sk] for l in layouts]).astype(np.int32)
    x, _, _ = make_case(78, B, H, Sq, Sk, D, dt, "single", q_off, k_off)
    scale = 1 / math.sqrt(D)
    o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = run_oracle(x, seg_q, seg_k, dt, scale, True, q_off, k_off)
    q, k, v, do = (to_dev(x[n], dt) for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o, lse, table = lwm.attention_forward(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, sq, sk, table, q_offset=q_off,
                                        k_offset=k_off)
    torch.cuda.synchronize()
    errs = [max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref), max_abs(f64(dq), dq_ref),
            max_abs(f64(dk), dk_ref), max_abs(f64(dv), dv_ref)]
    if dt == "bf16":
        od, lsed, _ = lwm.attention_decode(q, k, v, sq, sk, q_offset=q_off, k_offset=k_off, table=table)
        torch.cuda.synchronize()
        errs += [max_abs(f64(od), o_ref), max_abs(f64(lsed), lse_ref)]
    say("  max-abs O {:.2e} LSE {:.2e} dQ {:.2e} dK {:.2e} dV {:.2e}".format(*errs[:5])
        + (" decode O {:.2e} LSE {:.2e}".format(*errs[5:]) if dt == "bf16" else ""))
    assert np.array_equal(np.isinf(f64(lse)), np.isinf(lse_ref))
    tol_lse = TOL_LSE if dt == "bf16" else 1e-5
    assert errs[0] <= TOL_O[dt] and errs[1] <= tol_lse
    for n, g, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        check_grad(n, f64(g), r, dt)
    if dt == "bf16":
        assert errs[5] <= TOL_O[dt] and errs[6] <= TOL_LSE


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_rising_scores_rescale_every_tile(dt):
    """Scores that grow along the keys of each packed sample: each whole 64-key tile raises a
    row's running max by 1.3 times the lazy-update threshold (8 in log2 units), so the
    forward rescales its accumulator at most steps (all but a row's first and, when its
    diagonal sits early in a tile, its last).  Compared with the oracle element
    by element.  The backward is handed the stored O and forms Delta = <dO, O> from it, so
    its reference is the oracle's gradient given the same O: where a row's softmax sits on
    a few keys, dP - Delta is a small difference and the rounding of a bf16 O moves it by a
    visible share (with steeper slopes, LSE ~140, by about 8 % of max |dQ|)."""
    D = 128 if dt == "bf16" else 64
    S, H, seg_len = 1280, 2, 320
    say(f"rising scores {dt}: S={S} H={H} D={D} samples of {seg_len}")
    x, _, _ = make_case(51, 1, H, S, S, D, dt, "single")
    seg = (np.arange(S) // seg_len).astype(np.int32)[None]
    rng = np.random.default_rng(51)
    q = rng.normal(0, 0.5, (1, H, S, D)).astype(np.float32)
    k = rng.normal(0, 0.5, (1, H, S, D)).astype(np.float32)
    # score slope per key: 1.3 x the threshold (8 log2 units) per 64-key tile
    slope = 1.3 * 8 * math.log(2) * math.sqrt(D) / (40.0 * 64)
    q[..., 0] = 40.0
    k[..., 0] = slope * (np.arange(S) % seg_len)
    for n, arr in (("q", q), ("k", k)):
        x[n] = arr if dt == "f32" else li.bf16_bits_from_f32(arr)
    scale = 1 / math.sqrt(D)
    # the construction does what it is for: the running max jumps past the threshold at most
    # tile steps
    qh, kh, vh, doh = (host_f64(x[n], dt) for n in ("q", "k", "v", "do"))
    mask = A.visibility(seg[0], seg[0])
    s2 = np.where(mask, (qh[0, 0] @ kh[0, 0].T) * scale / math.log(2), -np.inf)
    tile_max = np.stack([s2[:, t:t + 64].max(axis=1) for t in range(0, S, 64)], axis=1)
    run_max = np.maximum.accumulate(tile_max, axis=1)
    live = np.isfinite(tile_max[:, 1:]) & np.isfinite(run_max[:, :-1])
    jumps = live & (tile_max[:, 1:] > run_max[:, :-1] + 8)
    assert jumps.sum() > 0.6 * live.sum()
    o_ref, lse_ref, _ = run_oracle(x, seg, seg, dt, scale, True, 0, 0, grads=False)
    qd, kd, vd, dod = (to_dev(x[n], dt) for n in ("q", "k", "v", "do"))
    sq = seg_dev(seg)
    o, lse, table = lwm.attention_forward(qd, kd, vd, sq, sq)
    dq, dk, dv = lwm.attention_backward(qd, kd, vd, o, dod, lse, sq, sq, table)
    torch.cuda.synchronize()
    eo, el = max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref)
    say(f"  max |LSE| {np.abs(lse_ref).max():.1f}; max-abs O {eo:.2e} LSE {el:.2e}")
    assert eo <= TOL_O[dt] and el <= TOL_LSE
    ref = A.backward(qh, kh, vh, doh, seg, seg, scale, True, o=f64(o))
    for n, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(n, f64(g), r, dt)


def test_backward_phases_on_two_streams():
    """The backward split into its phases: Delta on one stream, then dQ and dK/dV on two
    further streams that wait for it, running side by side; the gradients equal those of
    lwm_attn_bwd on one stream bit for bit (the phases share no scratch beyond Delta)."""
    B, H, S, D = 1, 4, 3000, 128
    say(f"backward phases on two streams: B={B} H={H} S={S}")
    x, seg_q, seg_k = make_case(61, B, H, S, S, D, "bf16", "packed")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    sq = seg_dev(seg_q)
    o, lse, table = lwm.attention_forward(q, k, v, sq, sq)
    desc = lwm.make_desc(B, H, S, S, D, torch.bfloat16)
    ws = torch.empty(lwm.lwm_attn_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(q) for _ in range(3)]
    lwm.lwm_attn_bwd(desc, q, k, v, o, do, lse, sq, sq, table, *ref, ws)
    torch.cuda.synchronize()
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws2 = torch.empty_like(ws)
    s0, s1, s2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    s0.wait_stream(torch.cuda.current_stream())
    lwm.lwm_attn_bwd_phase(desc, lwm.LWM_BWD_DELTA, q, k, v, o, do, lse, sq, sq, table, *got, ws2,
                           stream=s0)
    delta_done = torch.cuda.Event()
    delta_done.record(s0)
    for st, phase in ((s1, lwm.LWM_BWD_DQ), (s2, lwm.LWM_BWD_DKV)):
        st.wait_event(delta_done)
        lwm.lwm_attn_bwd_phase(desc, phase, q, k, v, o, do, lse, sq, sq, table, *got, ws2,
                               stream=st)
    torch.cuda.synchronize()
    same = [bool(torch.equal(g, r)) for g, r in zip(got, ref)]
    say(f"  dQ, dK, dV identical: {same}")
    assert all(same)
