"""Float64 packed-sequence loss reweighting: next-token cross-entropy in which every packed
sample carries the same total weight, and its gradient with respect to the logits.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source on the LWM pages: deep dive "LWM: million-token video-language world model", section
"Masked sequence packing": packing many samples into one sequence lets samples with many
tokens (long videos) outweigh samples with few loss tokens (short answers), so LWM reweights
the loss to match training the samples unpacked with padding (second step of its recipe;
the abstract page lists it as loss weighting, contribution (b)).  The pages give no formula;
the reading used: unpacked training with padding averages the loss over each sample's loss
tokens and then over the samples, so in the packed batch a loss token t of sample s gets
    w_t = 1 / (N * n_s),
with n_s the number of loss tokens of sample s and N the number of samples in the batch that
have at least one loss token.  Per token, with logits x_t (V values) and target y_t:
    l_t = logsumexp(x_t) - x_t[y_t],      loss = sum_t w_t l_t,
    d loss / d x_t = w_t (softmax(x_t) - onehot(y_t)),
times an upstream scalar gradient g.  A sample is identified by its segment id within its
batch row (ids need not be contiguous runs); a token is a loss token when its segment id is
>= 0 and its target is >= 0; other tokens have weight 0 and zero gradient.  With no loss
token at all the loss is 0.
"""
from __future__ import annotations

import numpy as np


def token_weights(targets, seg):
    """w [B,T] float64 from targets and segment ids [B,T]."""
    targets = np.asarray(targets)
    seg = np.asarray(seg)
    live = (seg >= 0) & (targets >= 0)
    counts = {}
    for b in range(seg.shape[0]):
        ids, n = np.unique(seg[b][live[b]], return_counts=True)
        for i, c in zip(ids, n):
            counts[(b, int(i))] = int(c)
    N = len(counts)
    w = np.zeros(seg.shape, np.float64)
    for (b, i), c in counts.items():
        w[b][(seg[b] == i) & live[b]] = 1.0 / (N * c)
    return w


def token_losses(logits, targets):
    """l [B,T] = logsumexp(x_t) - x_t[y_t] (0 where the target is negative)."""
    x = np.asarray(logits, np.float64)
    targets = np.asarray(targets)
    m = x.max(axis=-1, keepdims=True)
    lse = (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))[..., 0]
    y = np.where(targets >= 0, targets, 0)
    picked = np.take_along_axis(x, y[..., None], axis=-1)[..., 0]
    return np.where(targets >= 0, lse - picked, 0.0)


def token_grads(logits, targets, w, grad_scale=1.0):
    """dlogits [B,T,V] = grad_scale * w_t * (softmax(x_t) - onehot(y_t)) for given weights w
    (rows may be any subset of positions, with their weights from the whole batch)."""
    x = np.asarray(logits, np.float64)
    m = x.max(axis=-1, keepdims=True)
    p = np.exp(x - m)
    p /= p.sum(axis=-1, keepdims=True)
    targets = np.asarray(targets)
    onehot = np.zeros_like(p)
    b, t = np.nonzero(targets >= 0)
    onehot[b, t, targets[b, t]] = 1.0
    return (grad_scale * np.asarray(w, np.float64))[..., None] * (p - onehot)


def loss_and_grad(logits, targets, seg, grad_scale=1.0):
    """(loss, per-token loss l [B,T], dlogits [B,T,V]) in float64."""
    x = np.asarray(logits, np.float64)
    w = token_weights(targets, seg)
    l = token_losses(x, targets)
    loss = float(np.sum(w * l))
    return loss, l, token_grads(x, targets, w, grad_scale)
