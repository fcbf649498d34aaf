"""GPU parity of RoPE (lwm_attn_rope) with the float64 oracle (oracle/rope.py): every element
at small and medium sizes, forward and inverse, bf16 and float32, in place, positions up to
2^32 and theta from 1e4 to 5e7; then attention on rotated Q/K (forward and backward through
the rotation) against the oracle's composition, and sampled rows of the packed 128K
workload at the theta the pages give for 128K tokens.

The library stores rotated Q and K in the tensor's dtype, so for bf16 the attention reads
rotated values rounded to bf16.  The attention references round the oracle's float64
rotation the same way (nearest even) before the attention definition; without that step
the rounding alone moves LSE by about 2e-3 at 128K, beyond the 1e-3 bar."""
import math

import numpy as np
import pytest

import lwm_inputs as li
from oracle import attention as A
from oracle import rope as R
from gpu_helpers import TOL_GRAD, TOL_LSE, TOL_O, check_grad, f64, host_f64, max_abs, say, seg_dev, to_dev
from test_gpu_small import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lwm = pytest.importorskip("long_context_exact_blockwise_amd")


def stored(a64, dtype):
    """The rotated tensor as the library stores it: in the tensor's dtype (bf16 rounds to
    nearest even); attention then reads these rounded values."""
    if dtype != "bf16":
        return a64
    return li.bf16_bits_to_f64(li.bf16_bits_from_f32(np.asarray(a64, np.float32)))


def rope_error(y, ref, x, dtype):
    """Largest excess over the allowed error: bf16 results may be off by one bf16 unit in the
    last place (2^-8 relative) plus float32 rounding of the rotation; float32 results by a few
    float32 roundings of the pair's size."""
    pair = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    pair = np.repeat(pair, 2, axis=-1)
    if dtype == "bf16":
        tol = 2.0 ** -8 * np.abs(ref) + 2e-6 * pair
    else:
        tol = 1e-6 * pair + 1e-7
    return float(np.max(np.abs(y - ref) - tol)) if y.size else -1.0


CASES = [
    # name, seed, B, H, S, D, dtype, pos_offset, theta
    ("bf16_base", 1, 2, 3, 1000, 128, "bf16", 0, 1e4),
    ("bf16_1m_stage", 2, 1, 2, 777, 128, "bf16", (1 << 20) - 777, 5e7),
    ("bf16_128k_stage", 3, 1, 4, 300, 128, "bf16", 131072 - 300, 1e7),
    ("bf16_near_2p32", 4, 1, 1, 64, 128, "bf16", (1 << 32) - 64, 5e7),
    ("bf16_d16", 5, 1, 2, 333, 16, "bf16", 5000, 1e6),
    ("bf16_d256", 6, 1, 1, 129, 256, "bf16", 70000, 2.5e7),
    ("f32_d64", 7, 1, 2, 513, 64, "f32", 123456, 1e6),
    ("f32_d32", 8, 2, 1, 200, 32, "f32", (1 << 20) - 200, 5e7),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rope_matches_oracle(case):
    name, seed, B, H, S, D, dt, pos0, theta = case
    say(f"rope case {name}: B={B} H={H} S={S} D={D} {dt} pos0={pos0} theta={theta:g}")
    a = li.host_normal((B, H, S, D), seed, 1.0)
    xh = a if dt == "f32" else li.bf16_bits_from_f32(a)
    x64 = host_f64(xh, dt)
    pos = pos0 + np.arange(S)
    ref = R.rotate(x64, pos, theta)
    ref_inv = R.rotate(x64, pos, theta, inverse=True)
    x = to_dev(xh, dt)
    y = lwm.rope(x, pos0, theta)
    yi = lwm.rope(x, pos0, theta, inverse=True)
    xi = x.clone()
    lwm.rope(xi, pos0, theta, out=xi)  # in place
    torch.cuda.synchronize()
    e, ei = rope_error(f64(y), ref, x64, dt), rope_error(f64(yi), ref_inv, x64, dt)
    say(f"  max-abs {max_abs(f64(y), ref):.2e} (excess over bound {e:.1e}); inverse {ei:.1e}")
    assert e <= 0 and ei <= 0
    assert torch.equal(xi, y)
    assert np.array_equal(f64(x), x64)  # the source is untouched by the out-of-place calls


def test_rope_position_zero_is_exact_identity():
    say("rope: position 0 is the identity")
    x = to_dev(li.bf16_bits_from_f32(li.host_normal((1, 2, 1, 128), 9, 1.0)), "bf16")
    y = lwm.rope(x, 0, 5e7)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


ATT_CASES = [
    # name, seed, B, H, Sq, Sk, dtype, layout, q_off, k_off, theta
    ("bf16_packed", 21, 1, 2, 600, 600, "bf16", "packed", 0, 0, 1e7),
    ("bf16_chunk_offsets", 22, 1, 2, 384, 448, "bf16", "single", 900000, 899000, 5e7),
    ("f32_packed", 23, 1, 2, 300, 300, "f32", "packed", 0, 0, 1e6),
]


@pytest.mark.parametrize("case", ATT_CASES, ids=[c[0] for c in ATT_CASES])
def test_attention_with_rope_matches_oracle(case):
    name, seed, B, H, Sq, Sk, dt, layout, q_off, k_off, theta = case
    D = 128 if dt == "bf16" else 64
    say(f"rope attention case {name}: Sq={Sq} Sk={Sk} offs={q_off},{k_off} theta={theta:g} {dt}")
    x, seg_q, seg_k = make_case(seed, B, H, Sq, Sk, D, dt, layout, q_off, k_off)
    scale = 1 / math.sqrt(D)
    q, k, v, do = (host_f64(x[n], dt) for n in ("q", "k", "v", "do"))
    qpos, kpos = q_off + np.arange(Sq), k_off + np.arange(Sk)
    # the oracle's rotation, stored in the tensor dtype as the library stores it, then the
    # attention definition and the rotation back of dQ, dK (chain rule)
    qr, kr = stored(R.rotate(q, qpos, theta), dt), stored(R.rotate(k, kpos, theta), dt)
    o_ref, lse_ref = A.forward(qr, kr, v, seg_q, seg_k, scale, True, q_off, k_off)
    dqr, dkr, dv_ref = A.backward(qr, kr, v, do, seg_q, seg_k, scale, True, q_off, k_off)
    dq_ref = R.rotate(dqr, qpos, theta, inverse=True)
    dk_ref = R.rotate(dkr, kpos, theta, inverse=True)
    if dt == "f32":  # unrounded, this is exactly the oracle's composition
        o2, lse2 = R.attention_forward(q, k, v, seg_q, seg_k, scale, theta, True, q_off, k_off)
        assert max_abs(o2, o_ref) < 1e-12 and max_abs(lse2, lse_ref) < 1e-12
    qd, kd, vd, dod = (to_dev(x[n], dt) for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    o, lse, table = lwm.attention_forward(qd, kd, vd, sq, sk, q_offset=q_off, k_offset=k_off,
                                          rope_theta=theta)
    dq, dk, dv = lwm.attention_backward(qd, kd, vd, o, dod, lse, sq, sk, table, q_offset=q_off,
                                        k_offset=k_off, rope_theta=theta)
    torch.cuda.synchronize()
    eo, el = max_abs(f64(o), o_ref), max_abs(f64(lse), lse_ref)
    eq, ek, ev = max_abs(f64(dq), dq_ref), max_abs(f64(dk), dk_ref), max_abs(f64(dv), dv_ref)
    say(f"  max-abs O {eo:.2e} LSE {el:.2e} dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
    assert eo <= TOL_O[dt] and el <= TOL_LSE
    for n, g, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        check_grad(n, f64(g), r, dt)


def test_rope_packed_128k_sampled_rows():
    """RoPE at theta = 10M (the pages' 128K stage) on the packed 128K workload: the rotation of
    all Q and K rows against the oracle on 4 heads, then attention on the rotated tensors on
    sampled rows, each from its full masked score row."""
    w = li.WORKLOADS["packed_128k_fwd_bwd"]
    theta = 1e7
    segs = li.workload_segments(w)
    lengths = [n for _, n in segs]
    seg_q, seg_k = li.workload_segment_ids(w)
    say(f"{w.name}: RoPE theta {theta:g}, all rows of 4 heads, then sampled attention rows")
    q = li.device_normal((w.B, w.H, w.Sq, w.D), w.seed, w.value_scale, 0, torch.bfloat16, "cuda")
    k = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 1, torch.bfloat16, "cuda")
    v = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 2, torch.bfloat16, "cuda")
    qr, kr = lwm.rope(q, 0, theta), lwm.rope(k, 0, theta)
    o, lse, table = lwm.attention_forward(qr, kr, v, seg_dev(seg_q), seg_dev(seg_k))
    # RoPE inside the forward's Q load: the same bits as turning Q first
    o2, lse2, _ = lwm.attention_forward(q, k, v, seg_dev(seg_q), seg_dev(seg_k), table=table,
                                        rope_theta=theta)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    del o2, lse2
    pos = np.arange(w.Sq)
    worst_rot = -1.0
    samples = li.sample_rows(w, lengths)
    worst = [0.0, 0.0]
    for h, rows in samples.items():
        qh = q[0, h].float().cpu().numpy().astype(np.float64)
        kh = k[0, h].float().cpu().numpy().astype(np.float64)
        vh = v[0, h].float().cpu().numpy().astype(np.float64)
        qrh, krh = R.rotate(qh, pos, theta), R.rotate(kh, pos, theta)
        worst_rot = max(worst_rot, rope_error(f64(qr[0, h]), qrh, qh, "bf16"),
                        rope_error(f64(kr[0, h]), krh, kh, "bf16"))
        o_ref, lse_ref = A.forward_rows(stored(qrh[rows], "bf16"), stored(krh, "bf16"), vh,
                                        seg_q[0][rows], seg_k[0], rows, w.scale)
        worst[0] = max(worst[0], max_abs(f64(o[0, h])[rows], o_ref))
        worst[1] = max(worst[1], max_abs(f64(lse[0, h])[rows], lse_ref))
        del kh, vh, krh
    say(f"  rotation excess over bound {worst_rot:.1e}; sampled rows O {worst[0]:.2e} LSE {worst[1]:.2e}")
    assert worst_rot <= 0
    assert worst[0] <= TOL_O["bf16"] and worst[1] <= TOL_LSE


@pytest.mark.parametrize("case", [("packed", 31, 1, 2, 900, 900, 0, 0, 1e7, "packed"),
                                  ("ring_chunk_offsets", 32, 1, 1, 384, 448, 900000, 899000, 5e7, "single"),
                                  ("padded_b2", 33, 2, 2, 700, 700, 0, 0, 1e6, "padded")],
                         ids=["packed", "ring_chunk_offsets", "padded_b2"])
def test_rope_at_load_equals_rope_first(case):
    """lwm_attn_fwd_rope / lwm_attn_bwd_rope (Q or K turned inside the kernels' register
    loads) against lwm_attn_fwd / lwm_attn_bwd on tensors turned first by lwm_attn_rope: the
    turn at load rounds exactly as the standalone kernel, so O, LSE, the partial state and dV
    are identical bit for bit; dQ and dK are turned back in float32 before rounding instead
    of after, so they agree within bf16 rounding, and both against the oracle's composition."""
    name, seed, B, H, Sq, Sk, q_off, k_off, theta, layout = case
    say(f"rope at load, case {name}: B={B} H={H} Sq={Sq} Sk={Sk} offs={q_off},{k_off} theta={theta:g}")
    D = 128
    x, seg_q, seg_k = make_case(seed, B, H, Sq, Sk, D, "bf16", "single" if layout == "single" else "packed",
                                q_off, k_off, pad=layout == "padded")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    sq, sk = seg_dev(seg_q), seg_dev(seg_k)
    desc = lwm.make_desc(B, H, Sq, Sk, D, torch.bfloat16, q_offset=q_off, k_offset=k_off)
    table = lwm.lwm_attn_build_block_table(desc, sq, sk)
    qr, kr = lwm.rope(q, q_off, theta), lwm.rope(k, k_off, theta)
    o1, l1 = torch.empty_like(q), torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, qr, kr, v, sq, sk, table, o=o1, lse=l1)
    lwm.lwm_attn_fwd_rope(desc, lwm.LWM_OUT_FINAL, theta, q, kr, v, sq, sk, table, o=o2, lse=l2)
    st1 = lwm.attention_partial(qr, kr, v, sq, sk, q_offset=q_off, k_offset=k_off, table=table)
    st2 = tuple(torch.empty_like(t) for t in st1)
    lwm.lwm_attn_fwd_rope(desc, lwm.LWM_OUT_PARTIAL, theta, q, kr, v, sq, sk, table, m=st2[0], l=st2[1],
                          acc=st2[2])
    ws = torch.empty(lwm.lwm_attn_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    g1 = [torch.empty_like(t) for t in (q, k, v)]
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    lwm.lwm_attn_bwd(desc, qr, kr, v, o1, do, l1, sq, sk, table, *g1, ws)
    lwm.rope(g1[0], q_off, theta, inverse=True, out=g1[0])
    lwm.rope(g1[1], k_off, theta, inverse=True, out=g1[1])
    lwm.lwm_attn_bwd_rope(desc, theta, q, qr, k, kr, v, o2, do, l2, sq, sk, table, *g2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(st1, st2):
        assert torch.equal(a, b)
    assert torch.equal(g1[2], g2[2])
    e_unfused = [max_abs(f64(a), f64(b)) for a, b in zip(g1[:2], g2[:2])]
    say(f"  O, LSE, partial state, dV identical; dQ, dK vs turned-first path {e_unfused[0]:.1e} {e_unfused[1]:.1e}")
    # the oracle: attention on the turned inputs (rounded to bf16 as stored), gradients turned back
    scale = 1 / math.sqrt(D)
    qf, kf, vf, dof = (host_f64(x[n], "bf16") for n in ("q", "k", "v", "do"))
    qpos, kpos = q_off + np.arange(Sq), k_off + np.arange(Sk)
    qrf, krf = stored(R.rotate(qf, qpos, theta), "bf16"), stored(R.rotate(kf, kpos, theta), "bf16")
    dqr, dkr, dv_ref = A.backward(qrf, krf, vf, dof, seg_q, seg_k, scale, True, q_off, k_off)
    check_grad("dQ (RoPE at load)", f64(g2[0]), R.rotate(dqr, qpos, theta, inverse=True), "bf16")
    check_grad("dK (RoPE at load)", f64(g2[1]), R.rotate(dkr, kpos, theta, inverse=True), "bf16")
    check_grad("dV (RoPE at load)", f64(g2[2]), dv_ref, "bf16")
