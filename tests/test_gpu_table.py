"""GPU block table against the oracle's exact brute-force classification (integer work:
bit-exact where the table is exact, conservative where it may only be conservative)."""
import numpy as np
import pytest

import lwm_inputs as li
from oracle import table as otab
import test_oracle_pins as pins
from gpu_helpers import say, seg_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def gpu_table(seg_q, seg_k, Sq, Sk, bq, bk, q_off=0, k_off=0, causal=True):
    B = seg_q.shape[0]
    d = lwm.make_desc(B, 1, Sq, Sk, 128, torch.bfloat16, causal=causal, q_offset=q_off,
                      k_offset=k_off, block_q=bq, block_k=bk)
    t = lwm.lwm_attn_build_block_table(d, seg_dev(seg_q), seg_dev(seg_k))
    torch.cuda.synchronize()
    raw = t.cpu().numpy()
    nqb, nkb = -(-Sq // bq), -(-Sk // bk)
    al = lambda x: (x + 255) // 256 * 256
    qr_off, kr_off = 0, al(B * nqb * 8)
    st_off = kr_off + al(B * nkb * 8)
    q_rng = raw[qr_off:qr_off + B * nqb * 8].view(np.int32).reshape(B, nqb, 2)
    k_rng = raw[kr_off:kr_off + B * nkb * 8].view(np.int32).reshape(B, nkb, 2)
    st = raw[st_off:st_off + B * nqb * nkb].reshape(B, nqb, nkb)
    return st, q_rng, k_rng


def test_tiny_packed_table_is_the_hand_table():
    w = li.WORKLOADS["tiny_packed_f32"]
    sq, sk = li.workload_segment_ids(w)
    golden, _ = pins.load_golden_table()
    st, qr, kr = gpu_table(sq, sk, 256, 256, 64, 64)
    assert np.array_equal(st[0], golden)
    oq, ok = otab.ranges_from_status(golden)
    assert np.array_equal(qr[0], oq) and np.array_equal(kr[0], ok)


@pytest.mark.parametrize("seed", range(8))
def test_monotonic_layouts_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    Sq = int(rng.integers(1, 700))
    Sk = int(rng.integers(1, 700))
    bq = int(rng.choice([16, 32, 64]))
    bk = int(rng.choice([16, 32, 64]))
    causal = bool(seed % 4 != 3)
    q_off = int(rng.integers(0, 300)) if seed % 2 else 0
    k_off = int(rng.integers(0, 300)) if seed % 2 else 0
    total = max(q_off + Sq, k_off + Sk)
    ids = pins.random_layout(rng, total)
    sq = ids[q_off:q_off + Sq][None]
    sk = ids[k_off:k_off + Sk][None]
    say(f"table seed={seed} Sq={Sq} Sk={Sk} bq={bq} bk={bk} offs={q_off},{k_off} causal={causal}")
    st, qr, kr = gpu_table(sq, sk, Sq, Sk, bq, bk, q_off, k_off, causal)
    ref = otab.classify(sq[0], sk[0], bq, bk, q_off, k_off, causal)
    assert np.array_equal(st[0], ref)
    oq, ok = otab.ranges_from_status(ref)
    assert np.array_equal(qr[0], oq) and np.array_equal(kr[0], ok)


@pytest.mark.parametrize("seed", range(6))
def test_arbitrary_ids_conservative(seed):
    """Unordered ids with padding: SKIP must never hide a visible pair, FULL must be exact."""
    rng = np.random.default_rng(2000 + seed)
    B, Sq, Sk = 2, int(rng.integers(50, 500)), int(rng.integers(50, 500))
    sq = rng.integers(-1, 4, size=(B, Sq)).astype(np.int32)
    sk = rng.integers(-1, 4, size=(B, Sk)).astype(np.int32)
    sq[:, : Sq // 3] = 1  # give some blocks a single id so FULL can occur
    sk[:, : Sk // 3] = 1
    st, qr, kr = gpu_table(sq, sk, Sq, Sk, 32, 32, causal=bool(seed % 2))
    for b in range(B):
        ref = otab.classify(sq[b], sk[b], 32, 32, causal=bool(seed % 2))
        assert np.all(ref[st[b] == otab.SKIP] == otab.SKIP)
        assert np.array_equal(st[b] == otab.FULL, ref == otab.FULL)
        for a in range(ref.shape[0]):
            nz = np.nonzero(ref[a] != otab.SKIP)[0]
            if nz.size:
                assert qr[b, a, 0] <= nz[0] and qr[b, a, 1] >= nz[-1]


def test_ring_share_tables():
    """Chunked keys at global offsets: future chunks are all SKIP, past chunks all FULL."""
    chunk, n = 512, 8
    seg = np.zeros((1, chunk), np.int32)
    for c in range(n):
        st, qr, _ = gpu_table(seg, seg, chunk, chunk, 64, 64, q_off=5 * chunk, k_off=c * chunk)
        ref = otab.classify(seg[0], seg[0], 64, 64, 5 * chunk, c * chunk, True)
        assert np.array_equal(st[0], ref)
        if c > 5:
            assert np.all(st[0] == otab.SKIP) and np.all(qr[0, :, 1] < qr[0, :, 0])
        if c < 5:
            assert np.all(st[0] == otab.FULL)
