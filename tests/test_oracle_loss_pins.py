"""Pins of the float64 packed-loss oracle (oracle/packed_loss.py) against facts the pages and
mathematics fix: the packed loss equals unpacked training with padding (each sample's mean
token loss, averaged over samples), evaluated independently with torch's float64
cross-entropy and autograd; the uniform-logits closed form ln V; finite differences; and
the gradient's zero row sums."""
import math

import numpy as np
import pytest

from oracle import packed_loss as L

torch = pytest.importorskip("torch")


def packed_case(rng, lengths_per_row, V, ignore_frac=0.3):
    """Samples of the given lengths packed into rows (padding -1 to the longest row)."""
    T = max(sum(r) for r in lengths_per_row)
    B = len(lengths_per_row)
    seg = -np.ones((B, T), np.int64)
    targets = -np.ones((B, T), np.int64)
    for b, lens in enumerate(lengths_per_row):
        pos = 0
        for i, n in enumerate(lens):
            seg[b, pos:pos + n] = i
            t = rng.integers(0, V, n)
            t[rng.random(n) < ignore_frac] = -1  # tokens that are not loss tokens
            targets[b, pos:pos + n] = t
            pos += n
    logits = rng.standard_normal((B, T, V)) * 3.0
    return logits, targets, seg


def unpacked_reference(logits, targets, seg, lengths_per_row):
    """Each sample as its own padded batch row: torch cross-entropy (float64, ignore -1,
    mean over the sample's loss tokens), then the mean over samples with a loss token;
    gradients by autograd, mapped back to packed positions."""
    x = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    per_sample, where = [], []
    for b, lens in enumerate(lengths_per_row):
        pos = 0
        for n in lens:
            tg = torch.tensor(targets[b, pos:pos + n])
            if (tg >= 0).any():
                per_sample.append(torch.nn.functional.cross_entropy(x[b, pos:pos + n], tg,
                                                                    ignore_index=-1))
            pos += n
    loss = torch.stack(per_sample).mean() if per_sample else x.sum() * 0
    loss.backward()
    return float(loss.detach()), x.grad.numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_loss_equals_unpacked_training_with_padding(seed):
    rng = np.random.default_rng(seed)
    rows = [[5, 17, 3, 40], [2, 60], [9]]
    logits, targets, seg = packed_case(rng, rows, V=50)
    loss, _, grad = L.loss_and_grad(logits, targets, seg)
    ref_loss, ref_grad = unpacked_reference(logits, targets, seg, rows)
    assert abs(loss - ref_loss) < 1e-12
    assert np.max(np.abs(grad - ref_grad)) < 1e-14
    # and it is not the plain token mean (the samples have very different lengths)
    live = (seg >= 0) & (targets >= 0)
    token_mean = float(np.sum(L.token_losses(logits, targets) * live) / live.sum())
    assert abs(token_mean - loss) > 1e-3


def test_same_id_in_two_rows_is_two_samples():
    rng = np.random.default_rng(3)
    rows = [[30], [4]]
    logits, targets, seg = packed_case(rng, rows, V=20, ignore_frac=0.0)
    loss, _, _ = L.loss_and_grad(logits, targets, seg)
    ref_loss, _ = unpacked_reference(logits, targets, seg, rows)
    assert abs(loss - ref_loss) < 1e-12


def test_uniform_logits_give_ln_v():
    rng = np.random.default_rng(4)
    V = 37
    logits, targets, seg = packed_case(rng, [[6, 11], [25]], V)
    for level in (0.0, 1000.0, -1000.0):  # large offsets need the max shift to stay finite
        flat = np.full_like(logits, level)
        loss, l, grad = L.loss_and_grad(flat, targets, seg)
        assert abs(loss - math.log(V)) < 1e-12
        live = targets >= 0
        assert np.max(np.abs(l[live] - math.log(V))) < 1e-12


def test_gradient_by_finite_differences_and_zero_row_sums():
    rng = np.random.default_rng(5)
    rows = [[4, 7], [6]]
    logits, targets, seg = packed_case(rng, rows, V=9)
    g = 0.37
    loss, _, grad = L.loss_and_grad(logits, targets, seg, grad_scale=g)
    assert np.max(np.abs(grad.sum(axis=-1))) < 1e-15
    dead = (seg < 0) | (targets < 0)
    assert np.all(grad[dead] == 0)
    eps = 1e-6
    for idx in [(0, 0, 0), (0, 5, 3), (0, 10, 8), (1, 2, 4), (1, 5, 0)]:
        xp, xm = logits.copy(), logits.copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd = (L.loss_and_grad(xp, targets, seg)[0] - L.loss_and_grad(xm, targets, seg)[0]) / (2 * eps)
        assert abs(g * fd - grad[idx]) < 1e-8, (idx, fd, grad[idx])


def test_no_loss_token_gives_zero():
    rng = np.random.default_rng(6)
    logits, targets, seg = packed_case(rng, [[5, 5]], V=8)
    targets[:] = -1
    loss, l, grad = L.loss_and_grad(logits, targets, seg)
    assert loss == 0.0 and np.all(grad == 0) and np.all(l == 0)
