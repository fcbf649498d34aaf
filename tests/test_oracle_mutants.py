"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Each mutant replaces one oracle function for the duration of a test; the listed pins must
then fail.  This shows the pins constrain the parts of the oracle they are meant to.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))

from oracle import attention as A
from oracle import rope as R
import test_oracle_pins as pins
import test_oracle_rope_pins as rpins

_orig_visibility = A.visibility
_orig_backward_head = A.backward_head
_orig_merge = A.merge_states
_orig_forward_head = A.forward_head


def vis_strict_causal(seg_q, seg_k, q_offset=0, k_offset=0, causal=True):
    m = _orig_visibility(seg_q, seg_k, q_offset, k_offset, causal)
    if causal:
        qpos = q_offset + np.arange(len(seg_q))
        kpos = k_offset + np.arange(len(seg_k))
        m &= kpos[None, :] < qpos[:, None]
    return m


def vis_ignores_segments(seg_q, seg_k, q_offset=0, k_offset=0, causal=True):
    z = np.zeros(len(seg_q), np.int32), np.zeros(len(seg_k), np.int32)
    return _orig_visibility(z[0], z[1], q_offset, k_offset, causal)


def bwd_drops_delta(q, k, v, do, mask, scale):
    o, _, p = A.forward_head(q, k, v, mask, scale)
    dp = do @ v.T
    ds = p * dp
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def bwd_unscaled_dk(q, k, v, do, mask, scale):
    dq, dk, dv = _orig_backward_head(q, k, v, do, mask, scale)
    return dq, dk / scale, dv


def bwd_wrong_dv_operand(q, k, v, do, mask, scale):
    dq, dk, dv = _orig_backward_head(q, k, v, do, mask, scale)
    o, _, p = A.forward_head(q, k, v, mask, scale)
    return dq, dk, p.T @ o


def bwd_ignores_stored_o(q, k, v, do, mask, scale, o=None):
    # Delta always from the exact output, whatever output the backward is handed
    return _orig_backward_head(q, k, v, do, mask, scale)


def merge_same_weight(a, b):
    m1, l1, acc1 = a
    m2, l2, acc2 = b
    m = np.maximum(m1, m2)
    fin = np.isfinite(m)
    w = np.where(fin, np.exp(np.where(np.isfinite(m1), m1, 0) - np.where(fin, m, 0)), 0.0)
    w = np.where(np.isfinite(m1), w, 0.0)
    return np.where(fin, m, -np.inf), l1 * w + l2 * w, acc1 * w[:, None] + acc2 * w[:, None]


def fwd_lse_without_log(q, k, v, mask, scale):
    o, lse, p = _orig_forward_head(q, k, v, mask, scale)
    s = np.where(mask, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    return o, np.where(np.isfinite(lse), m + np.exp(lse - m), lse), p


_orig_rotate = R.rotate
_orig_rope_fwd = R.attention_forward


def rope_rotate_half_pairs(x, positions, theta, inverse=False):
    # pairs (x[i], x[i + D/2]) instead of (x[2i], x[2i+1])
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    perm = np.empty(x.shape[-1], np.int64)
    perm[0::2], perm[1::2] = np.arange(h), np.arange(h, 2 * h)
    inv = np.argsort(perm)
    return _orig_rotate(x[..., perm], positions, theta, inverse)[..., inv]


def rope_half_exponent(x, positions, theta, inverse=False):
    # frequencies theta^(-i/D) instead of theta^(-2i/D)
    return _orig_rotate(x, positions, float(theta) ** 0.5, inverse)


def rope_sign_flip(x, positions, theta, inverse=False):
    return _orig_rotate(x, positions, theta, not inverse)


def rope_bwd_no_unrotate(q, k, v, do, seg_q, seg_k, scale, theta, causal=True, q_offset=0,
                         k_offset=0):
    qr = _orig_rotate(q, q_offset + np.arange(q.shape[-2]), theta)
    kr = _orig_rotate(k, k_offset + np.arange(k.shape[-2]), theta)
    return A.backward(qr, kr, v, do, seg_q, seg_k, scale, causal, q_offset, k_offset)


def rope_fwd_local_key_positions(q, k, v, seg_q, seg_k, scale, theta, causal=True, q_offset=0,
                                 k_offset=0):
    qr = _orig_rotate(q, q_offset + np.arange(q.shape[-2]), theta)
    kr = _orig_rotate(k, np.arange(k.shape[-2]), theta)
    return A.forward(qr, kr, v, seg_q, seg_k, scale, causal, q_offset, k_offset)


def rope_fwd_local_query_positions(q, k, v, seg_q, seg_k, scale, theta, causal=True, q_offset=0,
                                   k_offset=0):
    qr = _orig_rotate(q, np.arange(q.shape[-2]), theta)
    kr = _orig_rotate(k, k_offset + np.arange(k.shape[-2]), theta)
    return A.forward(qr, kr, v, seg_q, seg_k, scale, causal, q_offset, k_offset)


ROPE_MUTANTS = [
    ("rotate", rope_rotate_half_pairs, [rpins.test_rope_worked_example]),
    ("rotate", rope_half_exponent, [rpins.test_rope_worked_example]),
    ("rotate", rope_sign_flip, [rpins.test_rope_worked_example]),
    ("attention_backward", rope_bwd_no_unrotate, [rpins.test_rope_attention_gradients_by_finite_differences]),
    ("attention_forward", rope_fwd_local_key_positions,
     [rpins.test_rope_attention_is_invariant_to_a_common_position_shift]),
    ("attention_forward", rope_fwd_local_query_positions,
     [rpins.test_rope_ring_chunks_with_global_key_positions_equal_full]),
]


@pytest.mark.parametrize("idx", range(len(ROPE_MUTANTS)))
def test_rope_pins_catch_mutant(idx, monkeypatch):
    name, mutant, checks = ROPE_MUTANTS[idx]
    monkeypatch.setattr(R, name, mutant)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


from oracle import packed_loss as PL
import test_oracle_loss_pins as lpins

_orig_weights = PL.token_weights
_orig_token_losses = PL.token_losses


def weights_token_mean(targets, seg):
    live = (np.asarray(seg) >= 0) & (np.asarray(targets) >= 0)
    return live / max(1, live.sum())


def weights_ids_shared_across_rows(targets, seg):
    # N and n_s counted per id over the whole batch, as if rows shared their samples
    seg = np.asarray(seg)
    live = (seg >= 0) & (np.asarray(targets) >= 0)
    ids, n = np.unique(seg[live], return_counts=True)
    w = np.zeros(seg.shape)
    for i, c in zip(ids, n):
        w[(seg == i) & live] = 1.0 / (len(ids) * c)
    return w


def losses_without_max_shift(logits, targets):
    x = np.asarray(logits, np.float64)
    targets = np.asarray(targets)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        lse = np.log(np.exp(x).sum(axis=-1))
    y = np.where(targets >= 0, targets, 0)
    picked = np.take_along_axis(x, y[..., None], axis=-1)[..., 0]
    return np.where(targets >= 0, lse - picked, 0.0)


def losses_shifted_target(logits, targets):
    t = np.asarray(targets)
    V = np.asarray(logits).shape[-1]
    return _orig_token_losses(logits, np.where(t >= 0, (t + 1) % V, t))


LOSS_MUTANTS = [
    ("token_weights", weights_token_mean,
     [lambda: lpins.test_packed_loss_equals_unpacked_training_with_padding(0)]),
    ("token_weights", weights_ids_shared_across_rows, [lpins.test_same_id_in_two_rows_is_two_samples]),
    ("token_losses", losses_without_max_shift, [lpins.test_uniform_logits_give_ln_v]),
    ("token_losses", losses_shifted_target,
     [lambda: lpins.test_packed_loss_equals_unpacked_training_with_padding(1)]),
]


@pytest.mark.parametrize("idx", range(len(LOSS_MUTANTS)))
def test_loss_pins_catch_mutant(idx, monkeypatch):
    name, mutant, checks = LOSS_MUTANTS[idx]
    monkeypatch.setattr(PL, name, mutant)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


from oracle import table as T

_orig_forward = A.forward
_orig_backward = A.backward
_orig_ranges = T.ranges_from_status


def fwd_batch_mask_of_row0(q, k, v, seg_q, seg_k, scale, causal=True, q_offset=0, k_offset=0):
    # every batch row attends under the first row's mask
    sq = np.repeat(np.asarray(seg_q)[:1], len(seg_q), axis=0)
    sk = np.repeat(np.asarray(seg_k)[:1], len(seg_k), axis=0)
    return _orig_forward(q, k, v, sq, sk, scale, causal, q_offset, k_offset)


def bwd_batch_do_of_row0(q, k, v, do, seg_q, seg_k, scale, causal=True, q_offset=0, k_offset=0):
    # the first row's upstream gradient reused for every batch row
    do0 = np.repeat(np.asarray(do)[:1], len(do), axis=0)
    return _orig_backward(q, k, v, do0, seg_q, seg_k, scale, causal, q_offset, k_offset)


def ranges_full_as_skip(status):
    st = np.where(np.asarray(status) == T.FULL, T.SKIP, status).astype(np.uint8)
    return _orig_ranges(st)


def ranges_last_one_short(status):
    q, k = _orig_ranges(status)
    q, k = q.copy(), k.copy()
    q[:, 1] = np.where(q[:, 1] > q[:, 0], q[:, 1] - 1, q[:, 1])
    k[:, 1] = np.where(k[:, 1] > k[:, 0], k[:, 1] - 1, k[:, 1])
    return q, k


def ranges_empty_as_zero(status):
    q, k = _orig_ranges(status)
    q, k = q.copy(), k.copy()
    q[q[:, 1] < q[:, 0]] = 0
    k[k[:, 1] < k[:, 0]] = 0
    return q, k


TABLE_MUTANTS = [
    ("ranges_from_status", ranges_full_as_skip, [lambda: pins.test_ranges_from_status_by_scanning(0)]),
    ("ranges_from_status", ranges_last_one_short, [pins.test_tiny_ranges_match_hand_derivation]),
    ("ranges_from_status", ranges_empty_as_zero, [lambda: pins.test_ranges_from_status_by_scanning(1)]),
]


@pytest.mark.parametrize("idx", range(len(TABLE_MUTANTS)))
def test_table_pins_catch_mutant(idx, monkeypatch):
    name, mutant, checks = TABLE_MUTANTS[idx]
    monkeypatch.setattr(T, name, mutant)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


MUTANTS = [
    ("forward", fwd_batch_mask_of_row0,
     [pins.test_batch_rows_equal_single_row_calls, pins.test_batch_matches_torch_sdpa_per_row_masks]),
    ("backward", bwd_batch_do_of_row0,
     [pins.test_batch_rows_equal_single_row_calls, pins.test_batch_matches_torch_sdpa_per_row_masks]),
    ("visibility", vis_strict_causal,
     [lambda: pins.test_brute_force_tiny(0), lambda: pins.test_matches_torch_sdpa_float64("single_causal")]),
    ("visibility", vis_ignores_segments,
     [lambda: pins.test_q_zero_gives_segment_prefix_mean(0), pins.test_packed_equals_per_segment]),
    ("backward_head", bwd_drops_delta, [pins.test_finite_difference_gradients]),
    ("backward_head", bwd_unscaled_dk, [pins.test_finite_difference_gradients]),
    ("backward_head", bwd_wrong_dv_operand, [pins.test_finite_difference_gradients]),
    ("backward_head", bwd_ignores_stored_o, [pins.test_stored_output_gradients_by_autograd]),
    ("merge_states", merge_same_weight, [pins.test_ring_order_merge_equals_full]),
    ("forward_head", fwd_lse_without_log,
     [lambda: pins.test_blockwise_equals_one_shot(64), lambda: pins.test_q_zero_gives_segment_prefix_mean(1)]),
]


@pytest.mark.parametrize("idx", range(len(MUTANTS)))
def test_pins_catch_mutant(idx, monkeypatch):
    name, mutant, checks = MUTANTS[idx]
    monkeypatch.setattr(A, name, mutant)
    for check in checks:
        with pytest.raises(AssertionError):
            check()
