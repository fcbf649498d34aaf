#!/usr/bin/env python3
"""Benchmark: exact blockwise causal attention, forward + backward, 131072 packed tokens.

One step is one pass of the whole path over one batch of synthetic input already resident
in HBM: build the block table from the segment ids, forward (O, LSE), backward (Delta, dQ,
dK, dV).  Throughput counts only unmasked FLOPs: 4*D per visible (query, key) pair per head
for the forward and 10*D for the backward (its five matmuls, including the recompute of
Q K^T), so 14*D for the step.

Prints one JSON line.  Beside the step time it reports each kernel's own time (HIP events
on the stream the library launches on), a roofline entry for the dominant kernel and the
float64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (unmasked FLOPs) fwd+bwd at 128K tokens; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
WORKLOAD = "packed_128k_fwd_bwd"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_packed_128k.json")
KERNEL_SOURCES = {
    "fwd": "attn_bf16.hip", "bwd_dq": "attn_bf16.hip", "bwd_dkv": "attn_bf16.hip",
    "bwd_delta": "attn_bf16.hip", "table": "table.hip",
}
# rocprofv3 kernel names of the kernels timed as parts
KERNEL_NAMES = {
    "fwd": "fwd_bf16_kernel", "bwd_dq": "dq_bf16_kernel", "bwd_dkv": "dkv_bf16_kernel",
    "bwd_delta": "delta_bf16_kernel",
}


def causal_pairs(lengths) -> int:
    """Visible (query, key) pairs of causal self-attention over packed segments."""
    return sum(n * (n + 1) // 2 for n in lengths)


def source_sha(name: str) -> str:
    path = os.path.join(ROOT, "long_context_exact_blockwise_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def time_events(fn, reps: int):
    """Average ms of fn() over reps, HIP events on torch's current stream (the stream the
    library launches on)."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps


def cpu_baseline(x_dev, lengths, scale, D, budget_s: float):
    """The float64 oracle, as it stands, on a 2048-token window starting at a segment start
    (a packed segment attends only to itself, so the window is an exact sub-instance),
    forward + backward, repeated over heads until `budget_s` seconds of CPU work."""
    import numpy as np

    import lwm_inputs as li
    from oracle import attention as A

    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = os.cpu_count() or 1
    bounds = li.segment_bounds(lengths)
    s0 = bounds[len(bounds) // 2][0]
    W = 2048
    seg = li.segment_ids_from_lengths(lengths)[s0:s0 + W][None]
    wlens = np.bincount(seg[0] - seg[0].min())
    pairs = causal_pairs([int(n) for n in wlens if n > 0])
    H = x_dev["q"].shape[1]
    heads_done, flops, t0 = 0, 0, time.perf_counter()
    while True:
        h = heads_done % H
        f = {n: x_dev[n][:, h:h + 1, s0:s0 + W].float().cpu().numpy().astype(np.float64)
             for n in ("q", "k", "v", "do")}
        t1 = time.perf_counter()
        A.forward(f["q"], f["k"], f["v"], seg, seg, scale)
        A.backward(f["q"], f["k"], f["v"], f["do"], seg, seg, scale)
        flops += 14 * D * pairs
        heads_done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    elapsed = time.perf_counter() - t0
    # the oracle forms the whole W x W masked score matrix; its dense rate counts every pair
    dense_flops = 14 * D * W * W * heads_done
    return {
        "value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "dense_value": dense_flops / elapsed / 1e12,
        "sample": f"NumPy float64 oracle, full masked score matrix, forward+backward of a "
                  f"{W}-token window at segment start {s0} of the same 131072-token packed "
                  f"layout, {heads_done} head(s), {elapsed:.1f} s; unmasked FLOPs (14*D per "
                  f"visible pair) / wall time",
        "cpu": cpu_model(),
        "blas": blas_name(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def blas_name() -> str:
    try:
        import numpy  # noqa: F401  (loads the BLAS threadpoolctl reports)
        import threadpoolctl

        for i in threadpoolctl.threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')}"
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return "unknown"


def decode_parts(lwm, li, torch, reps: int, unsplit: bool = False):
    """Split-KV decode against a 1M-token cache (one and sixteen new rows per head): the
    path streams K and V once, so it is priced against HBM bandwidth.  With `unsplit`, the
    plain forward on the same inputs is timed once beside it (kept out of the default run so
    that per-kernel profiles of the training forward see only its training launches)."""
    out = {}
    for name in ("decode_1m_q1", "decode_1m_q16"):
        w = li.WORKLOADS[name]
        seg_q, seg_k = li.workload_segment_ids(w)
        q = li.device_normal((w.B, w.H, w.Sq, w.D), w.seed, w.value_scale, 0, torch.bfloat16, "cuda")
        k = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 1, torch.bfloat16, "cuda")
        v = li.device_normal((w.B, w.H, w.Sk, w.D), w.seed, w.value_scale, 2, torch.bfloat16, "cuda")
        sq = torch.from_numpy(seg_q).cuda()
        sk = torch.from_numpy(seg_k).cuda()
        desc = lwm.make_desc(w.B, w.H, w.Sq, w.Sk, w.D, torch.bfloat16, q_offset=w.q_offset)
        table = lwm.lwm_attn_build_block_table(desc, sq, sk)
        ws = torch.empty(lwm.lwm_attn_decode_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
        ms = time_events(lambda: lwm.lwm_attn_decode(desc, q, k, v, sq, sk, table, o, lse, ws), reps)
        ms_unsplit = None
        if unsplit:  # the training forward on the same inputs: one workgroup per (tile, head)
            ms_unsplit = time_events(lambda: lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, q, k, v, sq, sk,
                                                              table, o=o, lse=lse), 1)
        # algorithmic bytes: K and V once, Q and O once, LSE
        algo = 2 * w.B * w.H * w.Sk * w.D * 2 + 2 * w.B * w.H * w.Sq * w.D * 2 + 4 * w.B * w.H * w.Sq
        gbs = algo / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "algo_bytes": algo, "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                     "workspace_bytes": ws.numel(), "unsplit_fwd_ms": ms_unsplit,
                     "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "q_offset": w.q_offset}
        print(f"[bench] {name}: {ms:.3f} ms, {gbs:.0f} GB/s"
              + (f" (unsplit forward {ms_unsplit:.2f} ms)" if ms_unsplit else ""), file=sys.stderr, flush=True)
        del q, k, v, o, lse, ws, table
    return out


def loss_part(lwm, li, torch, reps: int):
    """Packed-loss reweighting over the packed 128K workload's samples with a 40192-entry
    vocabulary: reads the bf16 logits once and writes their gradient once (HBM bound)."""
    import numpy as np

    w = li.WORKLOADS[WORKLOAD]
    V = 40192
    segs = li.workload_segments(w)
    seg = torch.from_numpy(li.segment_ids_from_lengths([n for _, n in segs])[None].astype(np.int32)).cuda()
    rng = np.random.default_rng(w.seed + 11)
    tg = torch.from_numpy(rng.integers(0, V, (1, w.Sq)).astype(np.int32)).cuda()
    x = li.device_normal((1, w.Sq, V), w.seed, 2.0, 5, torch.bfloat16, "cuda")
    dl = torch.empty_like(x)
    ws = torch.empty(lwm.lwm_attn_packed_loss_workspace_bytes(1, w.Sq, V, len(segs)), dtype=torch.uint8,
                     device="cuda")
    loss = torch.empty(4, dtype=torch.float32, device="cuda")
    ms = time_events(lambda: lwm.lwm_attn_packed_loss(x, tg, seg, len(segs), loss, None, dl, ws), reps)
    algo = 2 * x.numel() * 2 + w.Sq * 4 * 3
    gbs = algo / (ms * 1e-3) / 1e9
    print(f"[bench] packed loss 128K x {V}: {ms:.3f} ms, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    del x, dl
    return {"packed_loss_128k": {"ms": ms, "algo_bytes": algo, "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                                 "tokens": w.Sq, "vocab": V, "samples": len(segs)}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--part-reps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode and packed-loss parts")
    ap.add_argument("--decode-unsplit", action="store_true",
                    help="also time the plain forward on the decode inputs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (HBM counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU ring is not part of this build", file=sys.stderr)
        return 2

    import torch

    import long_context_exact_blockwise_amd as lwm
    import lwm_inputs as li

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        # a plain copy of known size: reads 1 GiB and writes 1 GiB per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 3}))
        return 0
    lwm.load_library()
    w = li.WORKLOADS[WORKLOAD]
    segs = li.workload_segments(w)
    lengths = [n for _, n in segs]
    seg_q, seg_k = li.workload_segment_ids(w)
    x = {n: li.device_normal((w.B, w.H, w.Sq, w.D), w.seed, w.grad_scale if n == "do" else w.value_scale,
                             i, torch.bfloat16, "cuda")
         for i, n in enumerate(("q", "k", "v", "do"))}
    sq = torch.from_numpy(seg_q).cuda()
    sk = torch.from_numpy(seg_k).cuda()
    desc = lwm.make_desc(w.B, w.H, w.Sq, w.Sk, w.D, torch.bfloat16, scale=w.scale, causal=True)
    table = torch.empty(lwm.lwm_attn_block_table_bytes(desc), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
    ws = torch.empty(lwm.lwm_attn_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")

    def step():
        lwm.lwm_attn_build_block_table(desc, sq, sk, table)
        lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, x["q"], x["k"], x["v"], sq, sk, table, o=o, lse=lse)
        lwm.lwm_attn_bwd(desc, x["q"], x["k"], x["v"], o, x["do"], lse, sq, sk, table, dq, dk, dv, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    print(f"[bench] {args.steps} steps, {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    pairs = causal_pairs(lengths)
    unit_flops = w.D * pairs * w.H * w.B  # D * (visible pairs over all heads)
    flops_step = 14 * unit_flops
    value = flops_step / (ms_step * 1e-3) / 1e12

    parts, roofline = {}, None
    if not args.no_parts:
        reps = args.part_reps
        ph = lambda p: (lambda: lwm.lwm_attn_bwd_phase(desc, p, x["q"], x["k"], x["v"], o, x["do"], lse,
                                                       sq, sk, table, dq, dk, dv, ws))
        parts["table"] = {"ms": time_events(lambda: lwm.lwm_attn_build_block_table(desc, sq, sk, table), reps)}
        parts["fwd"] = {"ms": time_events(lambda: lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, x["q"], x["k"],
                                                                   x["v"], sq, sk, table, o=o, lse=lse), reps),
                        "algo_flops": 4 * unit_flops}
        parts["bwd_delta"] = {"ms": time_events(ph(lwm.LWM_BWD_DELTA), reps),
                              "algo_bytes": (2 * w.D * 2 + 4) * w.B * w.H * w.Sq}
        parts["bwd_dq"] = {"ms": time_events(ph(lwm.LWM_BWD_DQ), reps), "algo_flops": 6 * unit_flops}
        parts["bwd_dkv"] = {"ms": time_events(ph(lwm.LWM_BWD_DKV), reps), "algo_flops": 8 * unit_flops}
        for k, p in parts.items():
            if "algo_flops" in p:
                p["tflops"] = p["algo_flops"] / (p["ms"] * 1e-3) / 1e12
                p["frac_peak"] = p["tflops"] / PEAK_BF16_TFLOPS
            if "algo_bytes" in p:
                p["gbs"] = p["algo_bytes"] / (p["ms"] * 1e-3) / 1e9
        # merge of two ring-share states (131072 query rows x 32 heads, D = 128)
        rows = 32 * 131072
        st = [torch.zeros((rows,), dtype=torch.float32, device="cuda") for _ in range(4)]
        accs = [torch.zeros((rows, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
        ms_merge = time_events(lambda: lwm.lwm_attn_merge_chunk(rows, 128, st[0], st[1], accs[0],
                                                                st[2], st[3], accs[1]), reps)
        merge_bytes = 12 * (128 + 2) * rows
        parts["merge_ring_state"] = {"ms": ms_merge, "algo_bytes": merge_bytes,
                                     "gbs": merge_bytes / (ms_merge * 1e-3) / 1e9,
                                     "frac_hbm_peak": merge_bytes / (ms_merge * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del st, accs
        # RoPE of Q and K at theta = 10M (the pages' 128K stage), each read and written once
        qr, kr = torch.empty_like(x["q"]), torch.empty_like(x["k"])
        ms_rope = time_events(lambda: (lwm.lwm_attn_rope(x["q"], qr, 0, 1e7),
                                       lwm.lwm_attn_rope(x["k"], kr, 0, 1e7)), reps)
        rope_bytes = 2 * 2 * x["q"].numel() * 2
        parts["rope_qk"] = {"ms": ms_rope, "algo_bytes": rope_bytes, "theta": 1e7,
                            "gbs": rope_bytes / (ms_rope * 1e-3) / 1e9,
                            "frac_hbm_peak": rope_bytes / (ms_rope * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del qr, kr
        dom = max(("fwd", "bwd_dq", "bwd_dkv"), key=lambda k: parts[k]["ms"])
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            tf = json.load(open(TRAFFIC_FILE))
            ent = tf.get(dom)
            if ent and ent.get("source_sha") == source_sha(KERNEL_SOURCES[dom]):
                traffic = ent.get("bytes_per_launch")
        roofline = {"bound": "mfma", "kernel": KERNEL_NAMES[dom],
                    "achieved": parts[dom]["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": parts[dom]["tflops"] / PEAK_BF16_TFLOPS, "traffic": traffic,
                    "avg_launch_ms": parts[dom]["ms"]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, lengths, w.scale, w.D, args.cpu_seconds)
        # extrapolations (not measured): the whole step on the CPU at the measured rates
        cpu["extrapolated_step_s_visible_pairs"] = flops_step / (cpu["value"] * 1e12)
        cpu["extrapolated_step_s_dense_matrix"] = (14 * w.D * w.Sq * w.Sq * w.H * w.B
                                                   / (cpu["dense_value"] * 1e12))

    if not args.no_parts and not args.no_decode:
        del x, o, lse, dq, dk, dv, ws, table
        parts.update(decode_parts(lwm, li, torch, args.part_reps, args.decode_unsplit))
        parts.update(loss_part(lwm, li, torch, args.part_reps))

    fwd_tflops = parts["fwd"]["tflops"] if parts else None
    bwd_ms = sum(parts[k]["ms"] for k in ("bwd_delta", "bwd_dq", "bwd_dkv")) if parts else None
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": w.B, "H": w.H, "D": w.D, "S": w.Sq,
                   "segments": len(segs), "seed": w.seed,
                   "visible_pairs_per_head": pairs,
                   "flops_per_step": flops_step,
                   "flop_count": "14*D per visible (query,key) pair per head: fwd 4*D + bwd 10*D"},
        "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
        # the same step counted as 12*D per pair (backward without the recompute of Q K^T)
        "value_12D_convention": value * 12 / 14,
        "fwd_tflops": fwd_tflops,
        "fwd_frac_of_peak": (fwd_tflops / PEAK_BF16_TFLOPS) if fwd_tflops else None,
        "bwd_tflops_10D": (10 * unit_flops / (bwd_ms * 1e-3) / 1e12) if bwd_ms else None,
        "parts": parts,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
