"""GPU parity of the packed-loss reweighting (lwm_attn_packed_loss) with the float64 oracle
(oracle/packed_loss.py): loss, per-token losses and every gradient element at small sizes
for each register-tile size, bf16 and float32 logits; then the packed 128K workload with an
LWM-sized vocabulary on sampled rows, the full-size weighting and reduction checked against
the oracle's weights, and the uniform-logits closed form on every row."""
import math

import numpy as np
import pytest

import lwm_inputs as li
from oracle import packed_loss as PL
from gpu_helpers import f64, host_f64, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def make_loss_case(seed, B, T, V, dtype, nseg, pad_tail=0, ignore_frac=0.3):
    rng = np.random.default_rng(seed)
    seg = np.sort(rng.integers(0, nseg, (B, T)), axis=1).astype(np.int32)
    if pad_tail:
        seg[:, T - pad_tail:] = -1
    tg = rng.integers(0, V, (B, T)).astype(np.int32)
    tg[rng.random((B, T)) < ignore_frac] = -1
    a = li.host_normal((B, T, V), seed, 3.0)
    x = a if dtype == "f32" else li.bf16_bits_from_f32(a)
    return x, tg, seg


def grad_excess(g, ref, w, dtype):
    wb = np.abs(w)[..., None]
    tol = (2.0 ** -8 * np.abs(ref) + 1e-6 * wb) if dtype == "bf16" else (1e-5 * wb + 1e-12)
    return float(np.max(np.abs(g - ref) - tol))


CASES = [
    # name, seed, B, T, V, dtype, nseg, pad_tail
    ("small_vocab_bf16", 1, 2, 300, 256, "bf16", 7, 20),
    ("small_vocab_f32", 2, 2, 300, 256, "f32", 7, 0),
    ("lwm_vocab_bf16", 3, 1, 96, 40192, "bf16", 5, 8),
    ("lwm_vocab_f32", 4, 1, 40, 40192, "f32", 3, 0),
    ("max_vocab_bf16", 5, 1, 12, 131072, "bf16", 2, 0),
    ("max_vocab_f32", 6, 1, 12, 65536, "f32", 2, 0),
    ("ragged_vocab_bf16", 7, 2, 50, 1000, "bf16", 4, 5),
    # one case per register tile the dispatch can pick (workgroup size x chunks per thread)
    ("tile256x8_bf16", 8, 1, 20, 16384, "bf16", 3, 0),
    ("tile256x16_llama_text_vocab_bf16", 9, 1, 20, 32000, "bf16", 3, 2),
    ("tile256x24_bf16", 10, 1, 20, 49152, "bf16", 3, 0),
    ("tile512x24_bf16", 11, 1, 16, 90000, "bf16", 3, 0),
    ("tile256x8_f32", 12, 1, 20, 16000, "f32", 3, 0),
    ("tile256x12_f32", 13, 1, 20, 24000, "f32", 3, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_packed_loss_matches_oracle(case):
    name, seed, B, T, V, dt, nseg, pad = case
    say(f"packed loss case {name}: B={B} T={T} V={V} {dt} samples/row<={nseg}")
    x, tg, seg = make_loss_case(seed, B, T, V, dt, nseg, pad)
    x64 = host_f64(x, dt)
    g = 0.5
    loss_ref, tl_ref, dl_ref = PL.loss_and_grad(x64, tg, seg, grad_scale=g)
    w = PL.token_weights(tg, seg)
    xd = to_dev(x, dt)
    tgd = torch.from_numpy(tg).cuda()
    segd = torch.from_numpy(seg).cuda()
    loss, tl, dl = lwm.packed_loss(xd, tgd, segd, nseg, grad_scale=g)
    loss2, _, _ = lwm.packed_loss(xd, tgd, segd, nseg, grad=False)
    torch.cuda.synchronize()
    el = abs(float(loss) - loss_ref)
    et = float(np.max(np.abs(f64(tl) - tl_ref)))
    eg = grad_excess(f64(dl), dl_ref, w, dt)
    say(f"  loss {float(loss):.6f} vs {loss_ref:.6f} (abs {el:.1e}); token loss {et:.1e}; "
        f"gradient excess over bound {eg:.1e}")
    assert el <= 1e-5 * max(1.0, abs(loss_ref)) and et <= 1e-4 and eg <= 0
    assert float(loss2) == float(loss)  # fixed-order sum: identical bits, with or without grad


def test_packed_loss_no_loss_token_and_empty_batch():
    say("packed loss: no loss token; empty batch")
    x = torch.zeros((1, 10, 64), dtype=torch.bfloat16, device="cuda")
    tg = -torch.ones((1, 10), dtype=torch.int32, device="cuda")
    seg = torch.zeros((1, 10), dtype=torch.int32, device="cuda")
    loss, tl, dl = lwm.packed_loss(x, tg, seg, 1)
    e = torch.empty((1, 0, 64), dtype=torch.bfloat16, device="cuda")
    ei = torch.empty((1, 0), dtype=torch.int32, device="cuda")
    loss0, _, _ = lwm.packed_loss(e, ei, ei, 1)
    torch.cuda.synchronize()
    assert float(loss) == 0.0 and torch.all(dl == 0) and torch.all(tl == 0)
    assert float(loss0) == 0.0


def test_packed_loss_128k_lwm_vocab():
    """The packed 128K workload's samples with a 40192-entry vocabulary (LLaMA-2's 32000 BPE ids
    plus 8192 VQGAN codes): text samples have 30% positions without loss (prompts), vision
    samples all count.  Sampled rows against the oracle; the loss against the oracle's
    weights applied to the kernel's own per-token losses (checks the weighting and the
    reduction over all 131072 positions); uniform logits give ln V exactly."""
    w = li.WORKLOADS["packed_128k_fwd_bwd"]
    V = 40192
    segs = li.workload_segments(w)
    seg = li.segment_ids_from_lengths([n for _, n in segs])[None].astype(np.int32)
    rng = np.random.default_rng(w.seed + 11)
    tg = rng.integers(0, V, (1, w.Sq)).astype(np.int32)
    for (kind, n), (s, e) in zip(segs, li.segment_bounds([n for _, n in segs])):
        if kind == "text":
            tg[0, s:e][rng.random(e - s) < 0.3] = -1
    say(f"packed loss 128K: {len(segs)} samples, V={V}")
    x = li.device_normal((1, w.Sq, V), w.seed, 2.0, 5, torch.bfloat16, "cuda")
    tgd, segd = torch.from_numpy(tg).cuda(), torch.from_numpy(seg).cuda()
    nseg = len(segs)
    loss, tl, dl = lwm.packed_loss(x, tgd, segd, nseg)
    torch.cuda.synchronize()
    wts = PL.token_weights(tg, seg)
    tl64 = f64(tl)
    # the kernel's reduction of its own token losses with the oracle's weights
    assert abs(float(loss) - float(np.sum(wts * tl64))) <= 1e-5 * abs(float(loss))
    rows = np.sort(rng.choice(w.Sq, 48, replace=False))
    rows = np.unique(np.concatenate([rows, [0, w.Sq - 1]]))
    xs = x[0, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)[None]
    tl_ref = PL.token_losses(xs, tg[:, rows])
    dl_ref = PL.token_grads(xs, tg[:, rows], wts[:, rows])  # weights from the whole sequence
    et = float(np.max(np.abs(tl64[0, rows] - tl_ref[0])))
    eg = grad_excess(f64(dl[0, torch.from_numpy(rows).cuda()])[None], dl_ref, wts[:, rows], "bf16")
    say(f"  loss {float(loss):.6f}; sampled rows: token loss {et:.1e}, gradient excess {eg:.1e}")
    assert et <= 1e-4 and eg <= 0
    del dl
    xz = torch.zeros_like(x)
    lz, _, _ = lwm.packed_loss(xz, tgd, segd, nseg, grad=False)
    torch.cuda.synchronize()
    say(f"  uniform logits: loss {float(lz):.7f} vs ln V {math.log(V):.7f}")
    assert abs(float(lz) - math.log(V)) <= 1e-5
