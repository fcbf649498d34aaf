"""Pins of the float64 oracle against facts fixed by the LWM pages and by mathematics.

None of these tests re-types the oracle's own formulas: each compares it with an
independent evaluation (pure-Python brute force, an online blockwise model written here,
per-segment attention, ring-order merging, closed forms, finite differences, torch's own
scaled-dot-product attention in float64) or with a hand-derived table.
"""
import math
import os

import numpy as np
import pytest

import lwm_inputs as li
import oracle
from oracle import attention as A
from oracle import brute, table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_case():
    w = li.WORKLOADS["tiny_packed_f32"]
    t = li.host_tensors(w)
    seg_q, seg_k = li.workload_segment_ids(w)
    f = lambda x: x[0, 0].astype(np.float64)
    return w, f(t["q"]), f(t["k"]), f(t["v"]), f(t["do"]), seg_q[0], seg_k[0]


def random_layout(rng, S, allow_padding=False):
    """Random contiguous segments; optionally a few padding (-1) tokens."""
    cuts = np.sort(rng.choice(np.arange(1, S), size=rng.integers(0, min(4, S - 1) + 1),
                              replace=False)) if S > 1 else np.array([], int)
    lengths = np.diff(np.concatenate([[0], cuts, [S]]))
    ids = li.segment_ids_from_lengths(lengths).astype(np.int32)
    if allow_padding:
        pad = rng.random(S) < 0.15
        ids = np.where(pad, -1, ids).astype(np.int32)
    return ids


# --------------------------------------------------------------------------------------
# 1. normalisation
# --------------------------------------------------------------------------------------

def test_rows_of_p_sum_to_one():
    w, q, k, v, do, sq, sk = tiny_case()
    mask = A.visibility(sq, sk)
    _, _, p = A.forward_head(q, k, v, mask, w.scale)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12)
    assert np.all(p[~mask] == 0.0)
    assert np.all(p >= 0.0)


# --------------------------------------------------------------------------------------
# 2. blockwise online softmax (the pages' "Blockwise Transformers" evaluation) == one shot
# --------------------------------------------------------------------------------------

def online_blockwise(q, k, v, mask, scale, block):
    """Key blocks visited in order; running max, denominator and accumulator per row."""
    Sq, D = q.shape[0], v.shape[1]
    m = np.full(Sq, -np.inf)
    l = np.zeros(Sq)
    acc = np.zeros((Sq, D))
    for j0 in range(0, k.shape[0], block):
        kb, vb, mb = k[j0:j0 + block], v[j0:j0 + block], mask[:, j0:j0 + block]
        s = scale * (q @ kb.T)
        s = np.where(mb, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0) - safe), 0.0)
        pblk = np.where(mb, np.exp(s - safe[:, None]), 0.0)
        l = alpha * l + pblk.sum(axis=1)
        acc = alpha[:, None] * acc + pblk @ vb
        m = m_new
    o = acc / l[:, None]
    return o, m + np.log(l)


@pytest.mark.parametrize("block", [1, 2, 3, 7, 64, 100, 256])
def test_blockwise_equals_one_shot(block):
    w, q, k, v, do, sq, sk = tiny_case()
    mask = A.visibility(sq, sk)
    o_ref, lse_ref, _ = A.forward_head(q, k, v, mask, w.scale)
    o, lse = online_blockwise(q, k, v, mask, w.scale, block)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


# --------------------------------------------------------------------------------------
# 3. masked packing: a packed batch == each segment attended alone
# --------------------------------------------------------------------------------------

def test_packed_equals_per_segment():
    w, q, k, v, do, sq, sk = tiny_case()
    mask = A.visibility(sq, sk)
    o, lse, _ = A.forward_head(q, k, v, mask, w.scale)
    dq, dk, dv = A.backward_head(q, k, v, do, mask, w.scale)
    for s, e in li.segment_bounds(li.FIXED3_LENGTHS):
        n = e - s
        causal = np.tril(np.ones((n, n), bool))
        o1, lse1, _ = A.forward_head(q[s:e], k[s:e], v[s:e], causal, w.scale)
        dq1, dk1, dv1 = A.backward_head(q[s:e], k[s:e], v[s:e], do[s:e], causal, w.scale)
        assert np.max(np.abs(o[s:e] - o1)) < 1e-12
        assert np.max(np.abs(lse[s:e] - lse1)) < 1e-12
        for g, g1 in ((dq, dq1), (dk, dk1), (dv, dv1)):
            assert np.max(np.abs(g[s:e] - g1)) < 1e-12


# --------------------------------------------------------------------------------------
# 4. ring: chunk states merged in ring order (and any order) == full attention
# --------------------------------------------------------------------------------------

def _ring_setup(seed=11, n_chunks=8, chunk=32, D=16, rank=5):
    rng = np.random.default_rng(seed)
    Sk = n_chunks * chunk
    q = rng.standard_normal((chunk, D))
    k = rng.standard_normal((Sk, D))
    v = rng.standard_normal((Sk, D))
    seg_all = np.zeros(Sk, np.int32)
    return q, k, v, seg_all, rank * chunk, chunk, n_chunks, D


def _chunk_state(q, k, v, seg_all, q_off, chunk, c, scale):
    ks = slice(c * chunk, (c + 1) * chunk)
    mask = A.visibility(seg_all[q_off:q_off + chunk], seg_all[ks], q_off, c * chunk, True)
    return A.partial_state(q, k[ks], v[ks], mask, scale)


def test_ring_order_merge_equals_full():
    q, k, v, seg_all, q_off, chunk, N, D = _ring_setup()
    scale = 1 / math.sqrt(D)
    full_mask = A.visibility(seg_all[q_off:q_off + chunk], seg_all, q_off, 0, True)
    o_ref, lse_ref, _ = A.forward_head(q, k, v, full_mask, scale)
    # device 5 holds chunk (5 - t) mod 8 at ring step t: 5, 4, 3, 2, 1, 0, 7, 6
    order = [(5 - t) % N for t in range(N)]
    assert order == [5, 4, 3, 2, 1, 0, 7, 6]
    rng = np.random.default_rng(3)
    for perm in [order] + [list(rng.permutation(N)) for _ in range(5)]:
        state = (np.full(chunk, -np.inf), np.zeros(chunk), np.zeros((chunk, D)))
        for c in perm:
            state = A.merge_states(state, _chunk_state(q, k, v, seg_all, q_off, chunk, c, scale))
        o, lse = A.finalize_state(state)
        assert np.max(np.abs(o - o_ref)) < 1e-12
        assert np.max(np.abs(lse - lse_ref)) < 1e-12


def test_future_chunks_are_empty_and_leave_state_unchanged():
    q, k, v, seg_all, q_off, chunk, N, D = _ring_setup()
    scale = 1 / math.sqrt(D)
    state = _chunk_state(q, k, v, seg_all, q_off, chunk, 5, scale)
    for c in (6, 7):
        st = _chunk_state(q, k, v, seg_all, q_off, chunk, c, scale)
        assert np.all(st[0] == -np.inf) and np.all(st[1] == 0) and np.all(st[2] == 0)
        merged = A.merge_states(state, st)
        for a, b in zip(merged, state):
            assert np.array_equal(a, b)
        merged = A.merge_states(st, state)
        for a, b in zip(merged, state):
            assert np.array_equal(a, b)


def test_two_empty_states_merge_to_empty():
    e = (np.full(3, -np.inf), np.zeros(3), np.zeros((3, 2)))
    m, l, acc = A.merge_states(e, e)
    assert np.all(m == -np.inf) and np.all(l == 0) and np.all(acc == 0)
    o, lse = A.finalize_state((m, l, acc))
    assert np.all(o == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------------------------
# 5. pure-Python brute force on tiny inputs
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    Sq = int(rng.integers(1, 13))
    Sk = int(rng.integers(1, 13))
    D = int(rng.integers(1, 5))
    causal = bool(rng.integers(0, 2))
    q_off = int(rng.integers(0, 6))
    k_off = int(rng.integers(0, 6))
    seg_q = random_layout(rng, Sq, allow_padding=True)
    seg_k = random_layout(rng, Sk, allow_padding=True)
    q = rng.standard_normal((Sq, D))
    k = rng.standard_normal((Sk, D))
    v = rng.standard_normal((Sk, D))
    do = rng.standard_normal((Sq, D))
    scale = 1 / math.sqrt(D)
    mask = A.visibility(seg_q, seg_k, q_off, k_off, causal)
    o, lse, _ = A.forward_head(q, k, v, mask, scale)
    ob, lseb = brute.forward(q.tolist(), k.tolist(), v.tolist(), seg_q.tolist(), seg_k.tolist(),
                             scale, causal, q_off, k_off)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    lseb = np.array(lseb)
    assert np.array_equal(np.isinf(lse), np.isinf(lseb))
    fin = np.isfinite(lse)
    assert np.max(np.abs(lse[fin] - lseb[fin]), initial=0) < 1e-12
    dq, dk, dv = A.backward_head(q, k, v, do, mask, scale)
    bq, bk, bv = brute.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), seg_q.tolist(),
                                seg_k.tolist(), scale, causal, q_off, k_off)
    for g, gb in ((dq, bq), (dk, bk), (dv, bv)):
        assert np.max(np.abs(g - np.array(gb))) < 1e-12


# --------------------------------------------------------------------------------------
# 6. closed forms
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q_zero_gives_segment_prefix_mean(seed):
    rng = np.random.default_rng(seed)
    S, D = 300, 8
    seg = random_layout(rng, S)
    v = rng.standard_normal((S, D))
    q = np.zeros((S, D))
    k = rng.standard_normal((S, D))
    o, lse, _ = A.forward_head(q, k, v, A.visibility(seg, seg), 0.125)
    # prefix sums restarted at each segment start
    csum = np.cumsum(v, axis=0)
    for i in range(S):
        start = i
        while start > 0 and seg[start - 1] == seg[i]:
            start -= 1
        n = i - start + 1
        mean = (csum[i] - (csum[start - 1] if start > 0 else 0)) / n
        assert np.max(np.abs(o[i] - mean)) < 1e-12
        assert abs(lse[i] - math.log(n)) < 1e-12


def test_q_zero_ring_offsets():
    """The same closed form with a query chunk at a global offset against all KV chunks."""
    rng = np.random.default_rng(5)
    chunk, N, D = 16, 4, 4
    q_off = 2 * chunk
    v = rng.standard_normal((N * chunk, D))
    k = rng.standard_normal((N * chunk, D))
    seg = np.zeros(N * chunk, np.int32)
    o, lse, _ = A.forward_head(np.zeros((chunk, D)), k, v,
                               A.visibility(seg[q_off:q_off + chunk], seg, q_off, 0), 0.5)
    for i in range(chunk):
        n = q_off + i + 1
        assert np.max(np.abs(o[i] - v[:n].mean(axis=0))) < 1e-12
        assert abs(lse[i] - math.log(n)) < 1e-12


def test_q_zero_backward_dv_closed_form():
    """With Q = 0, P_ij = 1/n_i on visible keys, so dV_j = sum over visible i of dO_i / n_i."""
    rng = np.random.default_rng(9)
    S, D = 40, 3
    seg = li.segment_ids_from_lengths([13, 20, 7])
    v = rng.standard_normal((S, D))
    k = rng.standard_normal((S, D))
    do = rng.standard_normal((S, D))
    _, _, dv = A.backward_head(np.zeros((S, D)), k, v, do, A.visibility(seg, seg), 0.3)
    bounds = li.segment_bounds([13, 20, 7])
    for s, e in bounds:
        for j in range(s, e):
            ref = sum(do[i] / (i - s + 1) for i in range(j, e))
            assert np.max(np.abs(dv[j] - ref)) < 1e-12


def test_single_token_segment():
    """A segment of one token sees only itself: O = v, LSE = its own score."""
    rng = np.random.default_rng(4)
    seg = li.segment_ids_from_lengths([5, 1, 6])
    q, k, v = (rng.standard_normal((12, 4)) for _ in range(3))
    o, lse, _ = A.forward_head(q, k, v, A.visibility(seg, seg), 0.7)
    assert np.max(np.abs(o[5] - v[5])) < 1e-15
    assert abs(lse[5] - 0.7 * float(q[5] @ k[5])) < 1e-14


def test_first_row_of_causal_segment_copies_value():
    rng = np.random.default_rng(8)
    seg = li.segment_ids_from_lengths([7, 9])
    q, k, v = (rng.standard_normal((16, 5)) for _ in range(3))
    o, _, _ = A.forward_head(q, k, v, A.visibility(seg, seg), 0.4)
    assert np.max(np.abs(o[0] - v[0])) < 1e-15
    assert np.max(np.abs(o[7] - v[7])) < 1e-15


# --------------------------------------------------------------------------------------
# 7. hand-derived block table of the tiny packed workload
# --------------------------------------------------------------------------------------

def load_golden_table():
    codes = {"S": table.SKIP, "P": table.PARTIAL, "F": table.FULL}
    rows, pairs = [], None
    with open(os.path.join(GOLDEN, "tiny_packed_table.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("pairs"):
                pairs = int(line.split()[1])
                continue
            if line.startswith(("q_range", "k_range")):
                continue
            rows.append([codes[c] for c in line.split()])
    return np.array(rows, np.uint8), pairs


def load_golden_ranges():
    """(q_range [nqb,2], k_range [nkb,2]) as read off the hand-derived table."""
    out = {}
    with open(os.path.join(GOLDEN, "tiny_packed_table.txt")) as f:
        for line in f:
            if line.startswith(("q_range", "k_range")):
                name, rest = line.split(None, 1)
                out[name] = np.array([[int(a) for a in part.split()] for part in rest.split("|")],
                                     np.int32)
    return out["q_range"], out["k_range"]


def test_tiny_table_matches_hand_derivation():
    w, q, k, v, do, sq, sk = tiny_case()
    golden, pairs = load_golden_table()
    st = table.classify(sq, sk, 64, 64)
    assert np.array_equal(st, golden)
    assert int((st == table.PARTIAL).sum()) == 7 and int((st == table.FULL).sum()) == 0
    assert table.visible_pairs(sq, sk) == pairs == 11356
    assert pairs * 4 * 64 == 2_907_136


def test_tiny_ranges_match_hand_derivation():
    """The per-row and per-column ranges of live tiles of the tiny packed table, read off by
    hand (tests/golden/tiny_packed_table.txt), equal the oracle's ranges_from_status."""
    w, q, k, v, do, sq, sk = tiny_case()
    q_gold, k_gold = load_golden_ranges()
    q_rng, k_rng = table.ranges_from_status(table.classify(sq, sk, 64, 64))
    assert np.array_equal(q_rng, q_gold)
    assert np.array_equal(k_rng, k_gold)


def _scan_ranges(status):
    """Independent evaluation by plain loops: walk each row (column) from both ends until a
    tile that is not SKIP is met; (0, -1) when the walk from the front runs off the end."""
    nqb, nkb = status.shape

    def walk(cells):
        n = len(cells)
        first = 0
        while first < n and cells[first] == table.SKIP:
            first += 1
        if first == n:
            return (0, -1)
        last = n - 1
        while cells[last] == table.SKIP:
            last -= 1
        return (first, last)

    q = [walk([int(status[a, c]) for c in range(nkb)]) for a in range(nqb)]
    k = [walk([int(status[a, c]) for a in range(nqb)]) for c in range(nkb)]
    return np.array(q, np.int32).reshape(nqb, 2), np.array(k, np.int32).reshape(nkb, 2)


@pytest.mark.parametrize("seed", range(6))
def test_ranges_from_status_by_scanning(seed):
    """Random status matrices (all three codes, whole empty rows and columns, 1 x n and n x 1
    shapes) and tables of random packed layouts with padding: ranges_from_status equals a
    scan from both ends of every row and column."""
    rng = np.random.default_rng(100 + seed)
    shapes = [(1, 7), (9, 1), (5, 5), (int(rng.integers(2, 12)), int(rng.integers(2, 12)))]
    mats = []
    for shp in shapes:
        st = rng.choice([table.SKIP, table.PARTIAL, table.FULL], size=shp,
                        p=[0.6, 0.25, 0.15]).astype(np.uint8)
        if shp[0] > 2:
            st[rng.integers(0, shp[0])] = table.SKIP      # an empty row
        if shp[1] > 2:
            st[:, rng.integers(0, shp[1])] = table.SKIP   # an empty column
        mats.append(st)
    S = int(rng.integers(100, 400))
    ids = random_layout(rng, S, allow_padding=True)
    ids[: int(rng.integers(0, 40))] = -1                  # leading padding: empty query blocks
    mats.append(table.classify(ids, ids, 16, 32))
    mats.append(table.classify(ids[:S // 2], ids, 32, 16, q_offset=S - S // 2, k_offset=0))
    for st in mats:
        q_rng, k_rng = table.ranges_from_status(st)
        q_ref, k_ref = _scan_ranges(st)
        assert np.array_equal(q_rng, q_ref), st
        assert np.array_equal(k_rng, k_ref), st


# --------------------------------------------------------------------------------------
# 8. gradients by central finite differences of L = <dO, O>
# --------------------------------------------------------------------------------------

def test_finite_difference_gradients():
    w, q, k, v, do, sq, sk = tiny_case()
    mask = A.visibility(sq, sk)
    dq, dk, dv = A.backward_head(q, k, v, do, mask, w.scale)
    rng = np.random.default_rng(21)
    h = 1e-6

    def loss(qq, kk, vv):
        o, _, _ = A.forward_head(qq, kk, vv, mask, w.scale)
        return float((do * o).sum())

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(12):
            i = int(rng.integers(0, 256))
            d = int(rng.integers(0, 64))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][i, d] += h
            lp = loss(args["q"], args["k"], args["v"])
            args[name][i, d] -= 2 * h
            lm = loss(args["q"], args["k"], args["v"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i, d]) <= 1e-6 * max(1.0, abs(grad[i, d])), (name, i, d)


def test_stored_output_gradients_by_autograd():
    """A backward handed a stored (rounded) output O': with c_i = <dO_i, O'_i - O_i> held
    fixed, its dQ and dK are torch autograd's float64 gradients of
    sum_i <dO_i, O_i> - sum_i c_i LSE_i (O and LSE formed by torch from the masked scores),
    and dV is unchanged; handed the exact O it gives the exact gradient."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(23)
    S, D, H = 80, 16, 2
    seg = li.segment_ids_from_lengths([30, 50])[None]
    q, k, v, do = (rng.standard_normal((1, H, S, D)) for _ in range(4))
    scale = 1 / math.sqrt(D)
    o, _ = A.forward(q, k, v, seg, seg, scale, True)
    exact = A.backward(q, k, v, do, seg, seg, scale, True)
    for g0, g1 in zip(exact, A.backward(q, k, v, do, seg, seg, scale, True, o=o)):
        assert np.max(np.abs(g0 - g1)) < 1e-13
    o_st = o + 0.05 * rng.standard_normal(o.shape)
    dq, dk, dv = A.backward(q, k, v, do, seg, seg, scale, True, o=o_st)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = torch.tensor(A.visibility(seg[0], seg[0], causal=True))
    s = (tq @ tk.transpose(-1, -2) * scale).masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    to = torch.exp(s - lse[..., None]) @ tv
    c = torch.tensor((do * (o_st - o)).sum(axis=-1))
    loss = (torch.tensor(do) * to).sum() - (c * lse).sum()
    loss.backward()
    for g, tg in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(g - tg.numpy())) < 1e-12
    # the stored output matters: the perturbation moves dQ
    assert np.max(np.abs(dq - exact[0])) > 1e-3


# --------------------------------------------------------------------------------------
# 9. special cases that reduce to a library routine: torch SDPA in float64 on the CPU
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["single_causal", "packed", "noncausal"])
def test_matches_torch_sdpa_float64(layout):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    rng = np.random.default_rng(17)
    S, D, H = 96, 16, 2
    if layout == "packed":
        seg = li.segment_ids_from_lengths([30, 41, 25])
        causal = True
    else:
        seg = np.zeros(S, np.int32)
        causal = layout == "single_causal"
    q, k, v, do = (rng.standard_normal((1, H, S, D)) for _ in range(4))
    scale = 1 / math.sqrt(D)
    o, lse = A.forward(q, k, v, seg[None], seg[None], scale, causal)
    dq, dk, dv = A.backward(q, k, v, do, seg[None], seg[None], scale, causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    if layout == "packed":
        allowed = torch.tensor((seg[:, None] == seg[None, :]) & np.tril(np.ones((S, S), bool)))
        to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
    else:
        to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do))
    assert np.max(np.abs(o - to.detach().numpy())) < 1e-12
    for g, tg in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(g - tg.numpy())) < 1e-12
    # LSE: logsumexp of the masked scores, by torch
    s = torch.tensor(q) @ torch.tensor(k).transpose(-1, -2) * scale
    m = torch.tensor(A.visibility(seg, seg, causal=causal))
    tl = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1)
    assert np.max(np.abs(lse - tl.numpy())) < 1e-12


# --------------------------------------------------------------------------------------
# 10. batches: each batch row with its own packing is its own instance
# --------------------------------------------------------------------------------------

def _batch_case(seed=29, B=3, H=2, Sq=70, Sk=90, D=8, q_off=20, k_off=0):
    rng = np.random.default_rng(seed)
    total = max(q_off + Sq, k_off + Sk)
    layouts = [random_layout(rng, total, allow_padding=False),
               random_layout(rng, total, allow_padding=True),
               np.zeros(total, np.int32)]
    layouts[0] = layouts[0] + 3                     # ids need not start at 0
    seg_q = np.stack([l[q_off:q_off + Sq] for l in layouts[:B]]).astype(np.int32)
    seg_k = np.stack([l[k_off:k_off + Sk] for l in layouts[:B]]).astype(np.int32)
    q = rng.standard_normal((B, H, Sq, D))
    k, v = rng.standard_normal((2, B, H, Sk, D))
    do = rng.standard_normal((B, H, Sq, D))
    return q, k, v, do, seg_q, seg_k, q_off, k_off


def test_batch_rows_equal_single_row_calls():
    """Three batch rows with different layouts (packed, padded, one segment) and their own
    values: the batched forward and backward equal each row run alone as a batch of one."""
    q, k, v, do, seg_q, seg_k, q_off, k_off = _batch_case()
    assert not np.array_equal(seg_q[0], seg_q[1]) and not np.array_equal(seg_q[1], seg_q[2])
    scale = 0.35
    o, lse = A.forward(q, k, v, seg_q, seg_k, scale, True, q_off, k_off)
    dq, dk, dv = A.backward(q, k, v, do, seg_q, seg_k, scale, True, q_off, k_off)
    for b in range(q.shape[0]):
        sl = slice(b, b + 1)
        ob, lb = A.forward(q[sl], k[sl], v[sl], seg_q[sl], seg_k[sl], scale, True, q_off, k_off)
        gb = A.backward(q[sl], k[sl], v[sl], do[sl], seg_q[sl], seg_k[sl], scale, True, q_off, k_off)
        assert np.array_equal(o[sl], ob) and np.array_equal(lse[sl], lb)
        for g, r in zip((dq, dk, dv), gb):
            assert np.array_equal(g[sl], r)


def test_batch_matches_torch_sdpa_per_row_masks():
    """The same batch against torch's float64 scaled-dot-product attention with a boolean
    mask per batch row (built here from the ids and global positions), forward and
    autograd; rows that see no key (padding) are checked to give O = 0 and LSE = -inf."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    q, k, v, do, seg_q, seg_k, q_off, k_off = _batch_case()
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    scale = 0.35
    o, lse = A.forward(q, k, v, seg_q, seg_k, scale, True, q_off, k_off)
    dq, dk, dv = A.backward(q, k, v, do, seg_q, seg_k, scale, True, q_off, k_off)
    allowed = np.zeros((B, 1, Sq, Sk), bool)
    for b in range(B):
        for i in range(Sq):
            for j in range(Sk):
                allowed[b, 0, i, j] = (seg_q[b, i] >= 0 and seg_q[b, i] == seg_k[b, j]
                                       and k_off + j <= q_off + i)
    live = allowed.any(axis=-1)[:, 0]                        # [B, Sq]
    assert (~live).any() and live.any()
    # torch gives NaN on rows with no visible key; feed it a harmless key for them and
    # zero their upstream gradient, then compare live rows only
    safe = allowed.copy()
    safe[..., 0] |= ~live[:, None, :]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(safe), scale=scale)
    to.backward(torch.tensor(do * live[:, None, :, None]))
    lv = live[:, None, :, None].repeat(H, 1)
    assert np.max(np.abs(np.where(lv, o - to.detach().numpy(), 0.0))) < 1e-12
    assert np.all(o[~lv.repeat(D, -1)] == 0.0)
    s = torch.tensor(q) @ torch.tensor(k).transpose(-1, -2) * scale
    tl = torch.logsumexp(s.masked_fill(~torch.tensor(safe), float("-inf")), dim=-1).numpy()
    l2 = live[:, None, :].repeat(H, 1)
    assert np.max(np.abs(np.where(l2, lse - tl, 0.0))) < 1e-12
    assert np.all(lse[~l2] == -np.inf)
    # gradients: rows that see nothing contribute nothing, so the oracle run on the same
    # upstream gradient restricted to live rows must match torch everywhere
    dq2, dk2, dv2 = A.backward(q, k, v, do * live[:, None, :, None], seg_q, seg_k, scale, True,
                               q_off, k_off)
    for g, tg in ((dq2, tq.grad), (dk2, tk.grad), (dv2, tv.grad)):
        assert np.max(np.abs(g - tg.numpy())) < 1e-12
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    assert np.max(np.abs(dq - dq2)) == 0.0


# --------------------------------------------------------------------------------------
# sampled-row forms agree with the full matrix
# --------------------------------------------------------------------------------------

def test_sampled_rows_agree_with_full():
    rng = np.random.default_rng(31)
    S, D = 200, 8
    seg = li.segment_ids_from_lengths([50, 70, 80])
    q, k, v, do = (rng.standard_normal((S, D)) for _ in range(4))
    mask = A.visibility(seg, seg)
    o, lse, _ = A.forward_head(q, k, v, mask, 0.3)
    dq, _, _ = A.backward_head(q, k, v, do, mask, 0.3)
    rows = np.array([0, 1, 49, 50, 51, 119, 120, 150, 199])
    orow, lrow = A.forward_rows(q[rows], k, v, seg[rows], seg, rows, 0.3, strip=4)
    assert np.max(np.abs(orow - o[rows])) < 1e-13
    assert np.max(np.abs(lrow - lse[rows])) < 1e-13
    dqr = A.dq_rows(q[rows], k, v, do[rows], seg[rows], seg, rows, 0.3, strip=4)
    assert np.max(np.abs(dqr - dq[rows])) < 1e-13
