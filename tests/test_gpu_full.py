"""GPU parity at the full workload sizes, through the same calls the benchmark times.

Outputs the oracle cannot form whole are checked on seeded sampled rows (each computed
exactly from its full masked score row), on whole sampled segments (a packed segment
attends only to itself, so the per-segment oracle is exact for it), on a 2048-token
sub-instance, on every row through the Q = 0 closed form (O = mean of V over the
visible keys, LSE = ln of their count), which checks the masks and the skip table
exhaustively, and on every head and segment through identities the exact gradient obeys."""
import math

import numpy as np
import pytest

import lwm_inputs as li
from oracle import attention as A
from gpu_helpers import TOL_GRAD, TOL_LSE, TOL_O, check_grad, f64, max_abs, say, seg_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def dev_inputs(w, names=("q", "k", "v"), Sk=None):
    out = {}
    for i, n in enumerate(("q", "k", "v", "do")):
        if n not in names:
            continue
        S = w.Sq if n in ("q", "do") else (w.Sk if Sk is None else Sk)
        sc = w.grad_scale if n == "do" else w.value_scale
        out[n] = li.device_normal((w.B, w.H, S, w.D), w.seed, sc, i, torch.bfloat16, "cuda")
    return out


def head_f64(t, b, h):
    return t[b, h].float().cpu().numpy().astype(np.float64)


def check_sampled_rows(w, x, o, lse, seg_q_np, seg_k_np, lengths, dq=None, k_offset=0,
                       k_full=None, v_full=None):
    """Forward (and dQ) of sampled rows against the oracle's per-row evaluation."""
    samples = li.sample_rows(w, lengths)
    worst = [0.0, 0.0, 0.0]
    dq_got, dq_all = [], []
    for h, rows in samples.items():
        qh = head_f64(x["q"], 0, h)[rows]
        kh = head_f64(k_full if k_full is not None else x["k"], 0, h)
        vh = head_f64(v_full if v_full is not None else x["v"], 0, h)
        pos = w.q_offset + rows
        o_ref, lse_ref = A.forward_rows(qh, kh, vh, seg_q_np[0][rows], seg_k_np[0], pos, w.scale,
                                        True, k_offset)
        worst[0] = max(worst[0], max_abs(f64(o[0, h])[rows], o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse[0, h])[rows], lse_ref))
        if dq is not None:
            doh = head_f64(x["do"], 0, h)[rows]
            dq_ref = A.dq_rows(qh, kh, vh, doh, seg_q_np[0][rows], seg_k_np[0], pos, w.scale,
                               True, k_offset)
            worst[2] = max(worst[2], max_abs(f64(dq[0, h])[rows], dq_ref))
            dq_got.append(f64(dq[0, h])[rows])
            dq_all.append(dq_ref)
    say(f"  sampled rows: max-abs O {worst[0]:.2e} LSE {worst[1]:.2e} dQ {worst[2]:.2e}")
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE and worst[2] <= TOL_GRAD["bf16"]
    if dq is not None:
        check_grad("dQ (sampled rows)", np.concatenate(dq_got), np.concatenate(dq_all), "bf16")


def q_zero_check(w, seg_ids, lengths, heads_for_o=2):
    """Forward with Q = 0 on the full workload; LSE on every row and head, O on a few heads."""
    x = dev_inputs(w, ("k", "v"))
    q = torch.zeros((w.B, w.H, w.Sq, w.D), dtype=torch.bfloat16, device="cuda")
    sq = seg_dev(seg_ids[None])
    o, lse, _ = lwm.attention_forward(q, x["k"], x["v"], sq, sq)
    torch.cuda.synchronize()
    cnt = np.zeros(w.Sq)
    for s, e in li.segment_bounds(lengths):
        cnt[s:e] = np.arange(1, e - s + 1)
    lse_all = f64(lse)[0]
    assert max_abs(lse_all, np.log(cnt)[None].repeat(w.H, 0)) <= TOL_LSE
    for h in (0, w.H - 1)[:heads_for_o]:
        vf = head_f64(x["v"], 0, h)
        ref = np.empty_like(vf)
        for s, e in li.segment_bounds(lengths):
            ref[s:e] = np.cumsum(vf[s:e], axis=0) / np.arange(1, e - s + 1)[:, None]
        assert max_abs(f64(o[0, h]), ref) <= TOL_O["bf16"]


def test_single_32k_sampled_rows():
    w = li.WORKLOADS["single_32k"]
    say(f"{w.name}: forward, {w.sample_heads}x{w.sample_rows_per_head} sampled rows")
    seg_q, seg_k = li.workload_segment_ids(w)
    lengths = [n for _, n in li.workload_segments(w)]
    x = dev_inputs(w)
    o, lse, _ = lwm.attention_forward(x["q"], x["k"], x["v"], seg_dev(seg_q), seg_dev(seg_k))
    torch.cuda.synchronize()
    check_sampled_rows(w, x, o, lse, seg_q, seg_k, lengths)


def test_single_32k_q_zero_all_rows():
    w = li.WORKLOADS["single_32k"]
    say(f"{w.name}: Q = 0 closed form, all rows")
    q_zero_check(w, li.workload_segment_ids(w)[0][0], [w.Sq])


def test_packed_64k_sampled_rows_and_q_zero():
    w = li.WORKLOADS["packed_64k"]
    segs = li.workload_segments(w)
    lengths = [n for _, n in segs]
    say(f"{w.name}: {len(segs)} segments; forward sampled rows + Q = 0 on all rows")
    seg_q, seg_k = li.workload_segment_ids(w)
    x = dev_inputs(w)
    o, lse, _ = lwm.attention_forward(x["q"], x["k"], x["v"], seg_dev(seg_q), seg_dev(seg_k))
    torch.cuda.synchronize()
    check_sampled_rows(w, x, o, lse, seg_q, seg_k, lengths)
    del x, o, lse
    q_zero_check(w, seg_q[0], lengths)


def test_ring_share_128k_x8_sampled_rows():
    w = li.WORKLOADS["ring_share_128k_x8"]
    chunk = w.Sk // w.n_chunks
    say(f"{w.name}: Q {w.Sq} at {w.q_offset} vs {w.n_chunks} chunks of {chunk}, ring order")
    seg_q, seg_k = li.workload_segment_ids(w)
    x = dev_inputs(w, ("q",))
    ks, vs, segs = [], [], []
    for c in range(w.n_chunks):
        ks.append(li.device_normal((w.B, w.H, chunk, w.D), w.seed * 100 + c, w.value_scale, 1,
                                   torch.bfloat16, "cuda"))
        vs.append(li.device_normal((w.B, w.H, chunk, w.D), w.seed * 100 + c, w.value_scale, 2,
                                   torch.bfloat16, "cuda"))
        segs.append(seg_dev(seg_k[:, c * chunk:(c + 1) * chunk]))
    order = lwm.ring_order(w.q_offset // chunk, w.n_chunks)
    o, lse, tables = lwm.ring_share_forward(x["q"], ks, vs, seg_dev(seg_q), segs,
                                            q_offset=w.q_offset,
                                            chunk_offsets=[c * chunk for c in range(w.n_chunks)],
                                            order=order)
    torch.cuda.synchronize()
    assert sorted(tables) == [0, 1, 2, 3, 4, 5]  # chunks 6 and 7 lie after every query
    samples = li.sample_rows(w, [w.Sk])
    worst = [0.0, 0.0]
    for h, rows in samples.items():
        qh = head_f64(x["q"], 0, h)[rows]
        kh = np.concatenate([head_f64(ks[c], 0, h) for c in range(w.n_chunks)])
        vh = np.concatenate([head_f64(vs[c], 0, h) for c in range(w.n_chunks)])
        o_ref, lse_ref = A.forward_rows(qh, kh, vh, seg_q[0][rows], seg_k[0], w.q_offset + rows,
                                        w.scale, True, 0)
        worst[0] = max(worst[0], max_abs(f64(o[0, h])[rows], o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse[0, h])[rows], lse_ref))
        del kh, vh
    say(f"  sampled rows: max-abs O {worst[0]:.2e} LSE {worst[1]:.2e}")
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE
    # Q = 0 on all rows: LSE = ln(q_offset + i + 1) for a single segment
    qz = torch.zeros_like(x["q"])
    _, lse0, _ = lwm.ring_share_forward(qz, ks, vs, seg_dev(seg_q), segs, q_offset=w.q_offset,
                                        chunk_offsets=[c * chunk for c in range(w.n_chunks)],
                                        order=order, tables=tables)
    torch.cuda.synchronize()
    cnt = np.log(w.q_offset + np.arange(w.Sq) + 1.0)
    assert max_abs(f64(lse0)[0], cnt[None].repeat(w.H, 0)) <= TOL_LSE


def test_packed_128k_fwd_bwd():
    w = li.WORKLOADS["packed_128k_fwd_bwd"]
    segs = li.workload_segments(w)
    lengths = [n for _, n in segs]
    bounds = li.segment_bounds(lengths)
    say(f"{w.name}: {len(segs)} segments; forward + backward at full size")
    seg_q, seg_k = li.workload_segment_ids(w)
    x = dev_inputs(w, ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o, lse, table = lwm.attention_forward(x["q"], x["k"], x["v"], sq, sk)
    dq, dk, dv = lwm.attention_backward(x["q"], x["k"], x["v"], o, x["do"], lse, sq, sk, table)
    torch.cuda.synchronize()
    check_sampled_rows(w, x, o, lse, seg_q, seg_k, lengths, dq=dq)
    # whole segments: dK, dV of every key of two seeded segments on two heads
    rng = np.random.default_rng(w.seed + 17)
    short = [i for i, (s, e) in enumerate(bounds) if e - s <= 4096]
    pick = rng.choice(short, size=min(2, len(short)), replace=False)
    heads = rng.choice(w.H, size=2, replace=False)
    worst = [0.0, 0.0, 0.0]
    for si in pick:
        s, e = bounds[si]
        causal = np.tril(np.ones((e - s, e - s), bool))
        for h in heads:
            qh, kh, vh, dh = (head_f64(x[n], 0, h)[s:e] for n in ("q", "k", "v", "do"))
            # the bf16 O the backward consumed enters only through Delta; the oracle uses its own
            dq_r, dk_r, dv_r = A.backward_head(qh, kh, vh, dh, causal, w.scale)
            say(f"  segment {si} [{s}, {e}) head {h}:")
            for i, (n, g, r) in enumerate((("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r))):
                worst[i] = max(worst[i], check_grad(n, f64(g[0, h])[s:e], r, "bf16")[0])
    say(f"  whole segments {list(pick)} heads {list(heads)}: dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")
    assert max(worst) <= TOL_GRAD["bf16"]
    check_gradient_identities(w, bounds, x, o, dq, dk, dv)


def check_gradient_identities(w, bounds, x, o, dq, dk, dv):
    """Identities of the exact gradient, on every head, segment and column at full size.
    Each row's weights sum to one over keys of its own segment and each row's dS sums to
    zero, so per segment sum_j dV_j = sum_i dO_i and sum_j dK_j = 0; and scaling q by c and
    k by 1/c leaves the scores unchanged, so per head sum_i <dQ_i, q_i> = sum_j <dK_j, k_j>.
    The GPU rounds P and dS to bf16 (relative 2^-9) before the products and its gradients to
    bf16 at the end, so each side may differ by 2^-9 of the sum of the magnitudes involved;
    the bars are twice that (2^-8)."""
    seg_idx = torch.empty(w.Sq, dtype=torch.long, device="cuda")
    for n, (s, e) in enumerate(bounds):
        seg_idx[s:e] = n

    def seg_sum(t):  # [B=1, H, S, D] -> float64 [segments, H, D]
        out = torch.zeros((len(bounds), w.H, w.D), dtype=torch.float64, device="cuda")
        return out.index_add_(0, seg_idx, t[0].double().transpose(0, 1))

    sv, so = seg_sum(dv), seg_sum(x["do"])
    tol_v = 2.0 ** -8 * (seg_sum(dv.abs()) + seg_sum(x["do"].abs())) + 1e-6
    rv = float(((sv - so).abs() / tol_v).max())
    sk = seg_sum(dk)
    # dS rounding: |sum_j d dS_ij| <= 2^-9 sum_j |dS_ij| <= 2^-9 * 2 |dO_i| max_j |v_j| per row
    rowfac = (x["do"].float().norm(dim=-1, keepdim=True) * x["q"].float().abs()).contiguous()
    vn = x["v"][0].float().norm(dim=-1).double()  # [H, S]
    vnorm_max = torch.stack([vn[:, s:e].amax(dim=1) for s, e in bounds])  # [segments, H]
    tol_k = 2.0 ** -8 * (seg_sum(dk.abs()) + w.scale * 2 * vnorm_max[..., None] * seg_sum(rowfac)) + 1e-6
    rk = float((sk.abs() / tol_k).max())
    lhs = (dq.double() * x["q"].double()).sum(dim=(2, 3))[0]
    rhs = (dk.double() * x["k"].double()).sum(dim=(2, 3))[0]
    mag = (dq.double() * x["q"].double()).abs().sum(dim=(2, 3))[0] + \
        (dk.double() * x["k"].double()).abs().sum(dim=(2, 3))[0]
    rq = float(((lhs - rhs).abs() / (2.0 ** -8 * mag)).max())
    say(f"  identities on all {w.H} heads, {len(bounds)} segments (error / bar, at most 1): "
        f"sum dV = sum dO {rv:.2e}, sum dK = 0 {rk:.2e}, <dQ, q> = <dK, k> {rq:.2e}")
    assert rv <= 1 and rk <= 1 and rq <= 1


def test_packed_128k_window_subinstance():
    """A 2048-token window starting at a segment start, run as its own instance and
    compared in full (forward and all gradients) on 8 heads."""
    w = li.WORKLOADS["packed_128k_fwd_bwd"]
    segs = li.workload_segments(w)
    lengths = [n for _, n in segs]
    bounds = li.segment_bounds(lengths)
    s0 = bounds[len(bounds) // 2][0]
    W, H = 2048, 8
    say(f"{w.name}: 2048-token window at segment start {s0}, {H} heads, full compare")
    seg_q, _ = li.workload_segment_ids(w)
    x = dev_inputs(w, ("q", "k", "v", "do"))
    win = {n: x[n][:, :H, s0:s0 + W].contiguous() for n in x}
    del x
    seg = seg_q[:, s0:s0 + W]
    sg = seg_dev(seg)
    o, lse, table = lwm.attention_forward(win["q"], win["k"], win["v"], sg, sg)
    dq, dk, dv = lwm.attention_backward(win["q"], win["k"], win["v"], o, win["do"], lse, sg, sg, table)
    torch.cuda.synchronize()
    hf = {n: f64(win[n]) for n in win}
    o_ref, lse_ref = A.forward(hf["q"], hf["k"], hf["v"], seg, seg, w.scale)
    g_ref = A.backward(hf["q"], hf["k"], hf["v"], hf["do"], seg, seg, w.scale)
    errs = [max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref)] + \
        [max_abs(f64(g), r) for g, r in zip((dq, dk, dv), g_ref)]
    say("  window max-abs O {:.2e} LSE {:.2e} dQ {:.2e} dK {:.2e} dV {:.2e}".format(*errs))
    assert errs[0] <= TOL_O["bf16"] and errs[1] <= TOL_LSE
    for n, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_ref):
        check_grad(n, f64(g), r, "bf16")


def test_packed_128k_closed_forms_all_rows():
    """Full-size closed forms on every row and key of the packed 128K workload:
    V = 1 gives O = 1 on every row (normalisation under random scores); Q = 0 gives uniform
    weights over the visible keys, so dK = 0 exactly (it is a multiple of Q) and
    dV_j = sum over later rows i of the segment of dO_i / n_i (n_i = keys row i sees), a
    suffix sum; both checked on every key of two heads, LSE = ln n_i on every row."""
    w = li.WORKLOADS["packed_128k_fwd_bwd"]
    segs = li.workload_segments(w)
    lengths = [n for _, n in segs]
    bounds = li.segment_bounds(lengths)
    say(f"{w.name}: closed forms on all rows (V = 1; Q = 0 forward + backward)")
    seg_q, seg_k = li.workload_segment_ids(w)
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    x = dev_inputs(w, ("q", "k", "do"))
    ones = torch.ones((w.B, w.H, w.Sk, w.D), dtype=torch.bfloat16, device="cuda")
    o1, _, _ = lwm.attention_forward(x["q"], x["k"], ones, sq, sk)
    torch.cuda.synchronize()
    err_one = float((o1.float() - 1.0).abs().max())
    del o1, ones
    v = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 2, torch.bfloat16, "cuda")
    q0 = torch.zeros_like(x["q"])
    o, lse, table = lwm.attention_forward(q0, x["k"], v, sq, sk)
    dq, dk, dv = lwm.attention_backward(q0, x["k"], v, o, x["do"], lse, sq, sk, table)
    torch.cuda.synchronize()
    cnt = np.zeros(w.Sq)
    for s, e in bounds:
        cnt[s:e] = np.arange(1, e - s + 1)
    err_lse = max_abs(f64(lse)[0], np.log(cnt)[None].repeat(w.H, 0))
    err_dk = float(dk.float().abs().max())
    err_dv = 0.0
    for h in (0, w.H - 1):
        dh = head_f64(x["do"], 0, h)
        ref = np.empty_like(dh)
        for s, e in bounds:
            wsum = dh[s:e] / cnt[s:e, None]
            ref[s:e] = np.cumsum(wsum[::-1], axis=0)[::-1]
        got = f64(dv[0, h])
        err_dv = max(err_dv, check_grad(f"dV(Q=0) head {h}", got, ref, "bf16")[0])
        # each segment on its own: a dV wrong or zero on the long tail of a segment, where the
        # suffix sums are small, fails the segment's relative error
        for s, e in bounds:
            check_grad(f"dV(Q=0) head {h} segment [{s}, {e})", got[s:e], ref[s:e], "bf16")
    say(f"  |O(V=1) - 1| {err_one:.2e}  LSE(Q=0) {err_lse:.2e}  |dK(Q=0)| {err_dk:.2e}  dV(Q=0) {err_dv:.2e}")
    assert err_one <= TOL_O["bf16"]
    assert err_lse <= TOL_LSE
    assert err_dk == 0.0
    assert err_dv <= TOL_GRAD["bf16"]


def test_long_single_segment_status_chunks():
    """A single causal segment of 147456 tokens (2304 tiles of 64, more than the 2048 tile
    classes a workgroup stages in LDS at a time), so the forward/dQ (last query tiles) and
    dK/dV (first key tiles) walk their tile range in two chunks.  Sampled rows of O, LSE and
    dQ against the oracle; Q = 0 closed forms on every row and key: LSE = ln(i + 1),
    dK = 0, dV by suffix sums."""
    S, H, D, seed = 147456, 2, 128, 41
    scale = 1 / math.sqrt(D)
    say(f"single segment S={S} H={H}: status staged in two chunks; sampled rows + Q = 0 closed forms")
    seg = torch.zeros((1, S), dtype=torch.int32, device="cuda")
    q, k, v, do = (li.device_normal((1, H, S, D), seed, 0.1 if i == 3 else 0.5, i, torch.bfloat16, "cuda")
                   for i in range(4))
    o, lse, table = lwm.attention_forward(q, k, v, seg, seg)
    dq, dk, dv = lwm.attention_backward(q, k, v, o, do, lse, seg, seg, table)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 63, 64, 131071, 131072, 140000, S - 65, S - 1],
                                     np.random.default_rng(seed).integers(0, S, 24)]))
    seg_np = np.zeros(S, np.int32)
    worst = [0.0, 0.0, 0.0]
    dq_got, dq_all = [], []
    for h in range(H):
        qh, kh, vh, dh = (head_f64(t, 0, h) for t in (q, k, v, do))
        o_ref, lse_ref = A.forward_rows(qh[rows], kh, vh, seg_np[rows], seg_np, rows, scale)
        dq_ref = A.dq_rows(qh[rows], kh, vh, dh[rows], seg_np[rows], seg_np, rows, scale)
        worst[0] = max(worst[0], max_abs(f64(o[0, h])[rows], o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse[0, h])[rows], lse_ref))
        worst[2] = max(worst[2], max_abs(f64(dq[0, h])[rows], dq_ref))
        dq_got.append(f64(dq[0, h])[rows])
        dq_all.append(dq_ref)
    say(f"  sampled rows: O {worst[0]:.2e} LSE {worst[1]:.2e} dQ {worst[2]:.2e}")
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE and worst[2] <= TOL_GRAD["bf16"]
    check_grad("dQ (sampled rows)", np.concatenate(dq_got), np.concatenate(dq_all), "bf16")
    del o, lse, dq, dk, dv
    q0 = torch.zeros_like(q)
    o, lse, table = lwm.attention_forward(q0, k, v, seg, seg, table=table)
    dq, dk, dv = lwm.attention_backward(q0, k, v, o, do, lse, seg, seg, table)
    torch.cuda.synchronize()
    cnt = np.arange(1, S + 1, dtype=np.float64)
    err_lse = max_abs(f64(lse)[0], np.log(cnt)[None].repeat(H, 0))
    err_dk = float(dk.float().abs().max())
    err_dv = 0.0
    for h in range(H):
        dh = head_f64(do, 0, h)
        ref = np.cumsum((dh / cnt[:, None])[::-1], axis=0)[::-1]
        got = f64(dv[0, h])
        err_dv = max(err_dv, check_grad(f"dV(Q=0) head {h}", got, ref, "bf16")[0])
        # the last quarter of the keys on its own (small suffix sums)
        check_grad(f"dV(Q=0) head {h} keys >= {3 * S // 4}", got[3 * S // 4:], ref[3 * S // 4:], "bf16")
    say(f"  Q = 0: LSE {err_lse:.2e} |dK| {err_dk:.2e} dV {err_dv:.2e}")
    assert err_lse <= TOL_LSE and err_dk == 0.0 and err_dv <= TOL_GRAD["bf16"]
