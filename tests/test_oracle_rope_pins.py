"""Pins of the float64 RoPE oracle (oracle/rope.py) against a hand-worked example and facts
of the rotation that any correct implementation must satisfy: pair norms kept, scores that
depend only on the difference of positions, inverse and composition, the D = 2 plane
rotation written as complex multiplication, the chain rule checked by finite differences,
and ring-order chunking with global key positions."""
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_worked_example():
    rows = []
    for line in open(os.path.join(GOLDEN, "rope_worked_example.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([float(t) for t in line.split()])
    return np.array(rows)


def test_rope_worked_example():
    ex = load_worked_example()
    x = np.array([[1.0, 2.0, 3.0, 4.0]] * len(ex))
    y = R.rotate(x, ex[:, 0], 100.0)
    assert np.max(np.abs(y - ex[:, 1:])) < 1e-14
    back = R.rotate(ex[:, 1:], ex[:, 0], 100.0, inverse=True)
    assert np.max(np.abs(back - x)) < 1e-14


def test_rope_keeps_every_pair_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 50, 128))
    pos = rng.integers(0, 1 << 20, 50)
    y = R.rotate(x, pos, 5e7)
    n_x = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_y = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(n_x - n_y)) < 1e-12


@pytest.mark.parametrize("theta", [1e4, 1e6, 5e7])
def test_rope_scores_depend_only_on_position_difference(theta):
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 40, 64))
    m = rng.integers(0, 4096, 40)
    n = rng.integers(0, 4096, 40)
    s0 = np.sum(R.rotate(q, m, theta) * R.rotate(k, n, theta), axis=1)
    for shift in (1, 777, 1 << 20):
        s1 = np.sum(R.rotate(q, m + shift, theta) * R.rotate(k, n + shift, theta), axis=1)
        assert np.max(np.abs(s1 - s0)) < 1e-8
    # and it does depend on the difference (theta is not degenerate)
    s2 = np.sum(R.rotate(q, m + 5, theta) * R.rotate(k, n, theta), axis=1)
    assert np.max(np.abs(s2 - s0)) > 1e-3


def test_rope_inverse_identity_and_composition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((30, 32))
    a = rng.uniform(0, 1e5, 30)
    b = rng.uniform(0, 1e5, 30)
    assert np.max(np.abs(R.rotate(R.rotate(x, a, 1e6), a, 1e6, inverse=True) - x)) < 1e-9
    assert np.max(np.abs(R.rotate(R.rotate(x, a, 1e6), b, 1e6) - R.rotate(x, a + b, 1e6))) < 1e-9
    assert np.array_equal(R.rotate(x, np.zeros(30), 1e6), x)


def test_rope_d2_is_complex_multiplication_by_unit_phase():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((25, 2))
    p = rng.integers(0, 100000, 25)
    z = (x[:, 0] + 1j * x[:, 1]) * np.exp(1j * p.astype(np.float64))  # frequency 1 for D = 2
    y = R.rotate(x, p, 5e7)
    assert np.max(np.abs(y[:, 0] - z.real)) < 1e-9 and np.max(np.abs(y[:, 1] - z.imag)) < 1e-9


def test_rope_attention_gradients_by_finite_differences():
    rng = np.random.default_rng(5)
    B, H, S, D = 1, 1, 12, 8
    q, k, v, do = (rng.standard_normal((B, H, S, D)) for _ in range(4))
    seg = np.zeros((B, S), np.int32)
    seg[0, 7:] = 1
    scale, theta, qo, ko = 0.4, 1e4, 300, 290

    def loss(q_, k_, v_):
        o, _ = R.attention_forward(q_, k_, v_, seg, seg, scale, theta, True, qo, ko)
        return float(np.sum(o * do))

    dq, dk, dv = R.attention_backward(q, k, v, do, seg, seg, scale, theta, True, qo, ko)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 3, 1), (0, 0, 8, 6), (0, 0, 11, 0), (0, 0, 0, 7)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-6, (name, idx, fd, g[idx])


def test_rope_ring_chunks_with_global_key_positions_equal_full():
    """Q at offset 256 against four KV chunks of 64 keys, each rotated at its own global
    offset and merged, equals the full forward."""
    rng = np.random.default_rng(6)
    D, theta, scale = 16, 5e7, 0.25
    q = rng.standard_normal((1, 1, 64, D))
    k, v = rng.standard_normal((2, 1, 1, 320, D))
    seg_q = np.zeros((1, 64), np.int32)
    seg_k = np.zeros((1, 320), np.int32)
    o_full, lse_full = R.attention_forward(q, k, v, seg_q, seg_k, scale, theta, True, 256, 0)
    qr = R.rotate(q, 256 + np.arange(64), theta)[0, 0]
    state = None
    for c in range(5):
        kr = R.rotate(k[0, 0, 64 * c:64 * (c + 1)], 64 * c + np.arange(64), theta)
        mask = A.visibility(seg_q[0], seg_k[0, 64 * c:64 * (c + 1)], 256, 64 * c, True)
        st = A.partial_state(qr, kr, v[0, 0, 64 * c:64 * (c + 1)], mask, scale)
        state = st if state is None else A.merge_states(state, st)
    o, lse = A.finalize_state(state)
    assert np.max(np.abs(o - o_full[0, 0])) < 1e-12 and np.max(np.abs(lse - lse_full[0, 0])) < 1e-12


def test_rope_packed_global_positions_equal_restarted_positions():
    """The stated reading: with packed samples, global positions give the same attention as
    positions that restart at every sample (scores depend on position differences only and
    samples never see each other)."""
    rng = np.random.default_rng(7)
    lengths = [30, 45, 25]
    S, D, theta, scale = sum(lengths), 32, 1e6, 0.2
    q, k, v = rng.standard_normal((3, 1, 1, S, D))
    seg = np.repeat(np.arange(3, dtype=np.int32), lengths)[None]
    o, lse = R.attention_forward(q, k, v, seg, seg, scale, theta)
    s0 = 0
    for n in lengths:
        sl = slice(s0, s0 + n)
        one = np.zeros((1, n), np.int32)
        o_s, lse_s = R.attention_forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], one, one, scale, theta)
        assert np.max(np.abs(o_s - o[:, :, sl])) < 1e-9 and np.max(np.abs(lse_s - lse[:, :, sl])) < 1e-9
        s0 += n


def test_rope_attention_is_invariant_to_a_common_position_shift():
    rng = np.random.default_rng(8)
    D, theta, scale = 16, 5e7, 0.25
    q = rng.standard_normal((1, 2, 40, D))
    k, v = rng.standard_normal((2, 1, 2, 70, D))
    seg_q = np.zeros((1, 40), np.int32)
    seg_k = np.zeros((1, 70), np.int32)
    o0, l0 = R.attention_forward(q, k, v, seg_q, seg_k, scale, theta, True, 50, 20)
    o1, l1 = R.attention_forward(q, k, v, seg_q, seg_k, scale, theta, True, 50 + 654321, 20 + 654321)
    assert np.max(np.abs(o1 - o0)) < 1e-8 and np.max(np.abs(l1 - l0)) < 1e-8
