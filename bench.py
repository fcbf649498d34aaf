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
import re
import sys
import time

import numpy as np

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


def _cpu_cores():
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        return max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        return os.cpu_count() or 1


def _run_for(budget_s: float, fn):
    """Call fn(i) for i = 0, 1, ... until budget_s seconds have passed (at least once);
    returns (calls, seconds, sum of what fn returned)."""
    n, acc, t0 = 0, 0, time.perf_counter()
    while True:
        acc += fn(n)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            return n, time.perf_counter() - t0, acc


def _tiled_normal(rows: int, D: int, seed: int, stream: int, scale: float = 0.5):
    """[rows, D] float64 from a seeded 8192-row block repeated: the oracle's work does not
    depend on the values, and drawing a 1M-row head afresh would cost more than timing it."""
    import numpy as np

    import lwm_inputs as li

    blk = li.host_normal((min(rows, 8192), D), seed, scale, stream).astype(np.float64)
    return np.tile(blk, (-(-rows // blk.shape[0]), 1))[:rows]


def cpu_baseline(x_dev, lengths, scale, D, budget_s: float):
    """The float64 oracle, as it stands, timed on bounded samples of the five workloads (each
    item runs whole units of work until its share of `budget_s` is spent):
      1. tiny packed fp32 (256 tokens, 3 segments, D = 64): full forward + backward;
      2. single 32K: sampled query rows (64 per head), each against its full masked row;
      3. 1M ring share: sampled query rows at global offset 5 * 131072 against all 1,048,576
         keys (values: a seeded 8192-row block repeated);
      4. packed 128K: forward + backward of a 2048-token window at a segment start (a packed
         segment attends only to itself, so the window is an exact sub-instance); the
         headline `value` (same workload and the same 14*D count as the GPU step);
      5. packed 128K: one head's forward in 256-row strips over the full masked
         131072-wide score matrix, strips spread evenly over the sequence.
    Rates count unmasked FLOPs (4*D per visible pair forward, 14*D forward + backward); the
    dense rate counts every pair of the masked matrices the oracle forms."""
    import numpy as np

    import lwm_inputs as li
    from oracle import attention as A

    share = {1: 0.05, 2: 0.12, 3: 0.25, 4: 0.33, 5: 0.25}
    items = {}

    # 1. tiny packed fp32, full
    w1 = li.WORKLOADS["tiny_packed_f32"]
    t1 = li.host_tensors(w1)
    f1 = {n: t1[n].astype(np.float64) for n in t1}
    s1q, s1k = li.workload_segment_ids(w1)
    p1 = causal_pairs(li.FIXED3_LENGTHS)

    def item1(_):
        A.forward(f1["q"], f1["k"], f1["v"], s1q, s1k, w1.scale)
        A.backward(f1["q"], f1["k"], f1["v"], f1["do"], s1q, s1k, w1.scale)
        return 1
    n, dt, _ = _run_for(budget_s * share[1], item1)
    items["tiny_packed_f32_full_fwd_bwd"] = {
        "tflops": 14 * w1.D * p1 * n / dt / 1e12, "dense_tflops": 14 * w1.D * 256 * 256 * n / dt / 1e12,
        "units": n, "unit": "full forward + backward", "seconds": dt}

    # 2. single 32K: 64 sampled rows per head, heads as the budget allows (8 planned)
    w2 = li.WORKLOADS["single_32k"]
    s2 = li.sample_rows(w2, [w2.Sq])
    seg2 = np.zeros(w2.Sq, np.int32)

    def item2(i):
        h, rows = list(s2.items())[i % len(s2)]
        k = _tiled_normal(w2.Sk, w2.D, w2.seed + h, 1)
        v = _tiled_normal(w2.Sk, w2.D, w2.seed + h, 2)
        q = _tiled_normal(w2.Sq, w2.D, w2.seed + h, 0)[rows]
        A.forward_rows(q, k, v, seg2[rows], seg2, rows, w2.scale)
        return int(np.sum(rows + 1))
    n, dt, pairs = _run_for(budget_s * share[2], item2)
    items["single_32k_sampled_rows_fwd"] = {
        "tflops": 4 * w2.D * pairs / dt / 1e12, "dense_tflops": 4 * w2.D * w2.Sk * 64 * n / dt / 1e12,
        "units": n, "unit": f"64 sampled rows of one head ({len(s2)} heads x 64 = 512 planned)",
        "seconds": dt}

    # 3. ring share: 64 sampled rows per head against all 1M keys (4 heads x 64 planned)
    w3 = li.WORKLOADS["ring_share_128k_x8"]
    s3 = li.sample_rows(w3, [w3.Sk])
    seg3 = np.zeros(w3.Sk, np.int32)

    def item3(i):
        h, rows = list(s3.items())[i % len(s3)]
        k = _tiled_normal(w3.Sk, w3.D, w3.seed + h, 1)
        v = _tiled_normal(w3.Sk, w3.D, w3.seed + h, 2)
        q = _tiled_normal(w3.Sq, w3.D, w3.seed + h, 0)[rows]
        pos = w3.q_offset + rows
        A.forward_rows(q, k, v, seg3[:w3.Sq][rows], seg3, pos, w3.scale)
        return int(np.sum(pos + 1))
    n, dt, pairs = _run_for(budget_s * share[3], item3)
    items["ring_share_1m_sampled_rows_fwd"] = {
        "tflops": 4 * w3.D * pairs / dt / 1e12, "dense_tflops": 4 * w3.D * w3.Sk * 64 * n / dt / 1e12,
        "units": n, "unit": f"64 sampled rows of one head against 1,048,576 keys ({len(s3)} heads planned)",
        "seconds": dt}

    # 4. packed 128K: 2048-token window at a segment start, forward + backward, head by head
    bounds = li.segment_bounds(lengths)
    s0 = bounds[len(bounds) // 2][0]
    W = 2048
    seg = li.segment_ids_from_lengths(lengths)[s0:s0 + W][None]
    wlens = np.bincount(seg[0] - seg[0].min())
    pairs4 = causal_pairs([int(n) for n in wlens if n > 0])
    H = x_dev["q"].shape[1]

    def item4(i):
        h = i % H
        f = {n: x_dev[n][:, h:h + 1, s0:s0 + W].float().cpu().numpy().astype(np.float64)
             for n in ("q", "k", "v", "do")}
        A.forward(f["q"], f["k"], f["v"], seg, seg, scale)
        A.backward(f["q"], f["k"], f["v"], f["do"], seg, seg, scale)
        return 1
    n4, dt4, _ = _run_for(budget_s * share[4], item4)
    value = 14 * D * pairs4 * n4 / dt4 / 1e12
    dense4 = 14 * D * W * W * n4 / dt4 / 1e12
    items["packed_128k_window_fwd_bwd"] = {
        "tflops": value, "dense_tflops": dense4, "units": n4,
        "unit": f"forward + backward of the {W}-token window at segment start {s0}, one head",
        "seconds": dt4}

    # 5. packed 128K: one head's forward in 256-row strips over the full masked matrix
    S5 = x_dev["q"].shape[2]
    ids5 = li.segment_ids_from_lengths(lengths)
    hq, hk, hv = (x_dev[n][0, 0].float().cpu().numpy().astype(np.float64) for n in ("q", "k", "v"))
    starts = np.arange(0, S5, 256)
    order = np.concatenate([starts[i::16] for i in range(16)])  # spread over the sequence
    seg_start = np.repeat([b[0] for b in bounds], [b[1] - b[0] for b in bounds])

    def item5(i):
        r0 = int(order[i % len(order)])
        rows = np.arange(r0, min(S5, r0 + 256))
        A.forward_rows(hq[rows], hk, hv, ids5[rows], ids5, rows, scale, strip=256)
        return int(np.sum(rows - seg_start[rows] + 1))
    n5, dt5, pairs5 = _run_for(budget_s * share[5], item5)
    items["packed_128k_head_strips_fwd"] = {
        "tflops": 4 * D * pairs5 / dt5 / 1e12, "dense_tflops": 4 * D * 256 * S5 * n5 / dt5 / 1e12,
        "units": n5, "unit": f"256-row strip of one head's full masked {S5}-wide score matrix "
                             f"({len(starts)} strips make the head)",
        "seconds": dt5,
        "extrapolated_full_head_fwd_s": dt5 / n5 * len(starts)}

    return {
        "value": value, "unit": "TFLOP/s", "cores": int(_cpu_cores()), "kind": "oracle",
        "dense_value": dense4,
        "sample": f"NumPy float64 oracle, full masked score matrix, forward+backward of a "
                  f"{W}-token window at segment start {s0} of the same 131072-token packed "
                  f"layout, {n4} head(s), {dt4:.1f} s; unmasked FLOPs (14*D per "
                  f"visible pair) / wall time; items lists the other four workloads' samples",
        "items": items,
        "budget_s": budget_s,
        "cpu": cpu_model(),
        "blas": blas_name(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


def rocminfo_peak():
    """The bf16 dense MFMA peak re-derived from what rocminfo reports for the gfx950 agent:
    compute units x max engine clock x 4096 flop per clock per CU (four SIMDs, each finishing
    one 32x32x16 bf16 MFMA, 32768 flop, every 32 clocks)."""
    import subprocess

    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception as e:  # pragma: no cover - rocminfo missing
        return {"error": f"rocminfo not run: {e}"}
    # one section per agent ("Agent N" ... ), each with its own Name / clock / CU lines; the
    # ISA entries nested in a GPU agent carry longer names (amdgcn-amd-amdhsa--gfx950...)
    agent = None
    for sec in re.split(r"\n(?=Agent \d+)", out):
        f = {}
        for line in sec.splitlines():
            k, _, v = line.strip().partition(":")
            if k in ("Name", "Compute Unit", "Max Clock Freq. (MHz)") and k not in f:
                f[k] = v.strip()
        if f.get("Name") == "gfx950" and "Compute Unit" in f and "Max Clock Freq. (MHz)" in f:
            agent = {"name": f["Name"], "cus": int(f["Compute Unit"]),
                     "mhz": int(f["Max Clock Freq. (MHz)"].split()[0])}
            break
    if agent is None:
        return {"error": "no gfx950 agent with compute units and clock in rocminfo output"}
    agent["flop_per_clk_per_cu"] = 4096
    agent["peak_tflops"] = agent["cus"] * agent["mhz"] * 1e6 * 4096 / 1e12
    return agent


def measured_gemm_tflops(torch, n: int = 16384, reps: int = 3):
    """A large bf16 GEMM through torch.matmul (hipBLASLt), HIP events: the practical ceiling
    of a dense contraction on this part, for context beside the published peak."""
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    ms = time_events(lambda: torch.matmul(a, b), reps)
    del a, b
    return {"n": n, "ms": ms, "tflops": 2 * n ** 3 / (ms * 1e-3) / 1e12, "reps": reps}


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


def median_events(torch, fn, reps: int, warmup: int = 3):
    """Median ms of fn() over reps runs, each bracketed by its own HIP events on torch's
    current stream, after `warmup` untimed runs."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2]


def config_table(lwm, li, torch, reps: int):
    """One JSON record per workload of the five: forward and backward kernel times (median of
    `reps` after 3 warm-ups, HIP events, inputs resident, block table built outside the timed
    region and timed on its own), TFLOP/s over unmasked FLOPs (4*D forward, 10*D backward per
    visible pair and head) and % of the published bf16 peak."""
    method = (f"median of {reps} runs after 3 warm-ups, HIP events on the launch stream, inputs "
              f"resident, block table built outside the timed region (timed separately)")
    for name in ("tiny_packed_f32", "single_32k", "packed_64k", "ring_share_128k_x8",
                 "packed_128k_fwd_bwd"):
        w = li.WORKLOADS[name]
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        rec = {"workload": name, "B": w.B, "H": w.H, "D": w.D, "Sq": w.Sq, "Sk": w.Sk,
               "dtype": w.dtype, "method": method}
        segs = li.workload_segments(w)
        lengths = [n for _, n in segs]
        seg_q, seg_k = li.workload_segment_ids(w)
        if name == "ring_share_128k_x8":
            chunk = w.Sk // w.n_chunks
            q = li.device_normal((w.B, w.H, w.Sq, w.D), w.seed, w.value_scale, 0, dt, "cuda")
            ks = [li.device_normal((w.B, w.H, chunk, w.D), w.seed * 100 + c, w.value_scale, 1, dt, "cuda")
                  for c in range(w.n_chunks)]
            vs = [li.device_normal((w.B, w.H, chunk, w.D), w.seed * 100 + c, w.value_scale, 2, dt, "cuda")
                  for c in range(w.n_chunks)]
            sq = torch.from_numpy(seg_q).cuda()
            sks = [torch.from_numpy(np.ascontiguousarray(seg_k[:, c * chunk:(c + 1) * chunk])).cuda()
                   for c in range(w.n_chunks)]
            offs = [c * chunk for c in range(w.n_chunks)]
            order = lwm.ring_order(w.q_offset // chunk, w.n_chunks)
            tables = {}
            t_tab = median_events(torch, lambda: [tables.update({c: lwm.lwm_attn_build_block_table(
                lwm.make_desc(w.B, w.H, w.Sq, chunk, w.D, dt, q_offset=w.q_offset, k_offset=offs[c]),
                sq, sks[c], tables.get(c))}) for c in order if offs[c] <= w.q_offset + w.Sq - 1], reps)
            mk = lambda: (torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda"),
                          torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda"),
                          torch.empty((w.B, w.H, w.Sq, w.D), dtype=torch.float32, device="cuda"))
            states = (mk(), mk())
            t_fwd = median_events(torch, lambda: lwm.ring_share_forward(
                q, ks, vs, sq, sks, q_offset=w.q_offset, chunk_offsets=offs, order=order,
                tables=tables, states=states), max(3, reps // 3))
            pairs = sum(w.q_offset + i + 1 for i in range(w.Sq))
            rec.update({"table_ms": t_tab, "fwd_ms": t_fwd, "visible_pairs_per_head": pairs,
                        "fwd_note": "6 chunk forwards (PARTIAL) + 5 merges + finalize, chunks 6, 7 skipped"})
            del q, ks, vs, states
        else:
            x = {n: li.device_normal((w.B, w.H, w.Sq if n in ("q", "do") else w.Sk, w.D), w.seed,
                                     w.grad_scale if n == "do" else w.value_scale, i, dt, "cuda")
                 for i, n in enumerate(("q", "k", "v", "do"))}
            sq, sk = torch.from_numpy(seg_q).cuda(), torch.from_numpy(seg_k).cuda()
            desc = lwm.make_desc(w.B, w.H, w.Sq, w.Sk, w.D, dt)
            table = torch.empty(lwm.lwm_attn_block_table_bytes(desc), dtype=torch.uint8, device="cuda")
            t_tab = median_events(torch, lambda: lwm.lwm_attn_build_block_table(desc, sq, sk, table), reps)
            o = torch.empty_like(x["q"])
            lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
            t_fwd = median_events(torch, lambda: lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, x["q"], x["k"],
                                                                  x["v"], sq, sk, table, o=o, lse=lse), reps)
            dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
            ws = torch.empty(max(lwm.lwm_attn_bwd_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
            t_bwd = median_events(torch, lambda: lwm.lwm_attn_bwd(desc, x["q"], x["k"], x["v"], o, x["do"], lse,
                                                                  sq, sk, table, dq, dk, dv, ws), reps)
            pairs = causal_pairs(lengths)
            rec.update({"table_ms": t_tab, "fwd_ms": t_fwd, "bwd_ms": t_bwd, "visible_pairs_per_head": pairs,
                        "segments": len(segs)})
            del x, o, lse, dq, dk, dv, ws, table
        unit = w.D * rec["visible_pairs_per_head"] * w.H * w.B
        rec["fwd_tflops"] = 4 * unit / (rec["fwd_ms"] * 1e-3) / 1e12
        rec["fwd_frac_of_peak"] = rec["fwd_tflops"] / PEAK_BF16_TFLOPS
        if "bwd_ms" in rec:
            rec["bwd_tflops_10D"] = 10 * unit / (rec["bwd_ms"] * 1e-3) / 1e12
            rec["fwd_bwd_ms"] = rec["fwd_ms"] + rec["bwd_ms"]
            rec["fwd_bwd_tflops_14D"] = 14 * unit / (rec["fwd_bwd_ms"] * 1e-3) / 1e12
            rec["fwd_bwd_frac_of_peak"] = rec["fwd_bwd_tflops_14D"] / PEAK_BF16_TFLOPS
        torch.cuda.empty_cache()
        print(json.dumps(rec), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--part-reps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode and packed-loss parts")
    ap.add_argument("--decode-unsplit", action="store_true",
                    help="also time the plain forward on the decode inputs")
    ap.add_argument("--probes", action="store_true",
                    help="only run the gfx950 microbenchmarks of tests/probes (one JSON record)")
    ap.add_argument("--configs", action="store_true",
                    help="only time each of the five workloads (one JSON record per workload)")
    ap.add_argument("--config-reps", type=int, default=10)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (HBM counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU ring transfer: a run measures one GPU's share", file=sys.stderr)
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
    if args.probes:
        sys.path.insert(0, os.path.join(ROOT, "tests", "probes"))
        import probes_lib

        print(json.dumps({"probes": probes_lib.run(torch)}), flush=True)
        return 0
    if args.configs:
        config_table(lwm, li, torch, args.config_reps)
        return 0
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
        # a training step with RoPE (theta = 10M): Q or K turned inside the attention kernels'
        # loads (K before the forward, Q and K before the backward: three streaming passes)
        # against turning Q and K first and dQ, dK back after (six passes)
        th = 1e7
        qr2, kr2 = torch.empty_like(x["q"]), torch.empty_like(x["k"])

        def rope_step_at_load():
            lwm.lwm_attn_rope(x["k"], kr, 0, th)
            lwm.lwm_attn_fwd_rope(desc, lwm.LWM_OUT_FINAL, th, x["q"], kr, x["v"], sq, sk, table, o=o, lse=lse)
            lwm.lwm_attn_rope(x["q"], qr2, 0, th)
            lwm.lwm_attn_rope(x["k"], kr2, 0, th)
            lwm.lwm_attn_bwd_rope(desc, th, x["q"], qr2, x["k"], kr2, x["v"], o, x["do"], lse, sq, sk,
                                  table, dq, dk, dv, ws)

        def rope_step_first():
            lwm.lwm_attn_rope(x["q"], qr, 0, th)
            lwm.lwm_attn_rope(x["k"], kr, 0, th)
            lwm.lwm_attn_fwd(desc, lwm.LWM_OUT_FINAL, qr, kr, x["v"], sq, sk, table, o=o, lse=lse)
            lwm.lwm_attn_rope(x["q"], qr2, 0, th)
            lwm.lwm_attn_rope(x["k"], kr2, 0, th)
            lwm.lwm_attn_bwd(desc, qr2, kr2, x["v"], o, x["do"], lse, sq, sk, table, dq, dk, dv, ws)
            lwm.lwm_attn_rope(dq, dq, 0, th, inverse=True)
            lwm.lwm_attn_rope(dk, dk, 0, th, inverse=True)

        parts["rope_step_at_load"] = {"ms": time_events(rope_step_at_load, reps), "theta": th,
                                      "note": "fwd + bwd with RoPE inside the kernels' loads, 3 RoPE passes"}
        parts["rope_step_turn_first"] = {"ms": time_events(rope_step_first, reps), "theta": th,
                                         "note": "fwd + bwd on Q, K turned first, dQ, dK turned back, 6 RoPE passes"}
        print(f"[bench] RoPE step: at load {parts['rope_step_at_load']['ms']:.3f} ms, turned first "
              f"{parts['rope_step_turn_first']['ms']:.3f} ms", file=sys.stderr, flush=True)
        del qr, kr, qr2, kr2
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

    peak_info = {"published_tflops": PEAK_BF16_TFLOPS, "rocminfo": rocminfo_peak()}
    if not args.no_parts:
        peak_info["gemm_bf16"] = measured_gemm_tflops(torch)
        print(f"[bench] bf16 GEMM 16384^3: {peak_info['gemm_bf16']['tflops']:.0f} TFLOP/s",
              file=sys.stderr, flush=True)
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
        "peak": peak_info,
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
