#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

Default workload: paged decode, batch 64, KV lengths uniform in [1, 4096],
64 query / 8 KV heads, head_dim 64, 16-token pages with a permuted page table
(the decode workload the headline metric is quoted on).  One step = one
pass of the decode path the library's automatic plan takes for it: the
load-balanced first pass (sink_attn_decode_balanced_partial, every wave
streaming an equal share of the batch's pages) followed by its finish pass
(sink_attn_decode_balanced_finish, the LSE merge of requests that span
several ranges), both through the C ABI.  Metric: KV bytes read per second
(2 * Hkv * 64 * 2 B per KV token) over the whole step.  --decode-plan
chunked times the split-KV pair (sink_attn_decode_partial +
sink_attn_merge) instead.

Also reported, on the same JSON line:
  * "roofline": the dominant kernel (the first pass) -- algorithmic bytes
    per launch / its mean launch time from HIP events around it on its own
    stream (every fourth launch of the timed region), against the 8 TB/s
    HBM peak; "traffic" from rocprofv3 counters when a measurement for the
    current kernel exists, else null;
  * "prefill": the causal prefill workload (8 x 4096 tokens, 64/8 heads,
    contiguous KV) in TFLOP/s against the 2.5 PFLOP/s dense bf16 peak;
  * "cpu_baseline": the fp64 oracle timed on this host's cores on the same
    decode batch.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --mode traffic   # kernels only, for rocprofv3 --pmc passes

--mode traffic runs, untimed: a plain 256 MiB device-to-device copy three
times (the calibration dispatch for FETCH_SIZE / WRITE_SIZE), then the decode
first pass eight times on the decode workload (rotating the same four KV
copies as the timed run), then the prefill kernel three times.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
KV_COPIES = 4                  # rotated KV pools: 4 x 269 MB > 256 MB last-level cache
EVENT_EVERY = 4                # timed decode steps between two sampled first-pass launches

# HBM bytes per dispatch from rocprofv3 FETCH_SIZE + WRITE_SIZE passes
# (python bench.py --mode traffic), each scaled by the same counter on a
# 256 MiB copy; see profiles/.  Valid for the kernel sources they were taken
# on -- reset to None whenever decode_balanced.hip or prefill.hip changes.
DECODE_TRAFFIC_BYTES = 260_946_607
PREFILL_TRAFFIC_BYTES = 1_871_242_272


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def decode_algorithmic_bytes(b) -> int:
    """Bytes the definition must read once: K and V of every KV token
    (2 * Hkv * D * 2 B each), the queries, page ids and per-request lengths."""
    L = b.kv_len.astype(np.int64)
    kv = int(L.sum()) * 2 * b.num_kv_heads * b.head_dim * 2
    q = int(b.qo_indptr[-1]) * b.num_qo_heads * b.head_dim * 2   # query rows
    pages = int(((L + b.page_size - 1) // b.page_size).sum()) * 4
    return kv + q + pages + b.batch * 8


def prefill_pairs(b) -> int:
    """Unmasked (query row, head, key) triples of a causal prefill."""
    qlens = np.diff(b.qo_indptr).astype(np.int64)
    kvl = b.kv_len.astype(np.int64)
    # query t sees keys 0 .. kv_len - qlen + t  ->  sum_t (kv_len - qlen + t + 1)
    per_req = qlens * (kvl - qlens) + qlens * (qlens + 1) // 2
    return int(per_req.sum()) * b.num_qo_heads


def bench_decode(args, torch, sa, device, W):
    b = W.config(2)
    balanced = args.decode_plan == "balanced"
    db = device.to_device(b, plan="balanced" if balanced else "chunked")
    B, Hq, D = db.batch, db.num_qo_heads, db.head_dim
    out_code = sa.F32 if db.out.dtype == torch.float32 else sa.BF16
    if balanced:
        R = sa.sink_attn_decode_num_ranges(B, db.num_kv_heads, db.max_kv_len, 0)
        plan = dict(num_ranges=R)
    else:
        S = device.splits_of(db)
        o_parts = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
        lse_parts = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        plan = dict(num_splits=S)
    ks = [db.k] + [db.k.clone() for _ in range(KV_COPIES - 1)]
    vs = [db.v] + [db.v.clone() for _ in range(KV_COPIES - 1)]
    torch.cuda.synchronize()

    def first(k, v):
        if balanced:
            sa.sink_attn_decode_balanced_partial(
                db.q, k, v, db.kv_indptr, db.page_indices, db.kv_len, db.sinks, B, Hq,
                db.num_kv_heads, D, db.page_size, db.max_kv_len, 0, db.sm_scale, db.out,
                out_code, db.lse, db.workspace, db.workspace_bytes)
        else:
            sa.sink_attn_decode_partial(db.q, k, v, db.kv_indptr, db.page_indices, db.kv_len,
                                        db.sinks, B, Hq, db.num_kv_heads, D, db.page_size,
                                        db.max_kv_len, db.num_splits, db.sm_scale, o_parts,
                                        lse_parts)

    def second():
        if balanced:
            sa.sink_attn_decode_balanced_finish(db.kv_indptr, db.sinks, B, Hq, db.num_kv_heads, D,
                                                db.max_kv_len, 0, db.out, out_code, db.lse,
                                                db.workspace, db.workspace_bytes)
        else:
            sa.sink_attn_merge(o_parts, lse_parts, B, Hq, S, D, db.out, out_code, db.lse)

    def step(i, ev=None):
        k, v = ks[i % KV_COPIES], vs[i % KV_COPIES]
        if ev is not None:
            ev[0].record()
        first(k, v)
        if ev is not None:
            ev[1].record()
        second()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The first pass is bracketed by events on every EVENT_EVERY-th step of
    # the timed region: each pair of event records costs the stream a few
    # microseconds, which would otherwise be charged to every step.
    sampled = [i for i in range(args.steps) if i % EVENT_EVERY == 0]
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in sampled}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i, evs.get(i))
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    kern_ms = float(np.mean([a.elapsed_time(c) for a, c in evs.values()]))
    kv_bytes = int(b.kv_len.astype(np.int64).sum()) * 2 * b.num_kv_heads * b.head_dim * 2
    alg = decode_algorithmic_bytes(b)
    ms_step = total_ms / args.steps
    res = dict(batch=b, db=db, plan=plan, ms_step=ms_step, kern_ms=kern_ms,
               kern_samples=len(evs), kv_bytes=kv_bytes,
               alg_bytes=alg, value=kv_bytes / (ms_step * 1e-3) / 1e9, first=first)
    return res


def _time_calls(torch, fn, steps, warmup):
    """Mean ms of fn(i) over `steps` calls, HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(c) for a, c in evs]))


def kv_bytes_of(b) -> int:
    return int(b.kv_len.astype(np.int64).sum()) * 2 * b.num_kv_heads * b.head_dim * 2


def bench_extra(args, torch, sa, device, W):
    """The other workloads, each timed whole (all kernels of the call), HIP
    events: the long split decode (workload 3), both calls of the mixed batch
    (workload 5), a multi-token verification batch (64 requests, 4 drafted
    tokens each, KV lengths U[4, 4096]) through sink_attn_prefill and
    sink_attn_verify, and 16-token drafts (linear, then random trees) through
    sink_attn_verify and sink_attn_verify_tree, the bias + rotary +
    paged-append step on a prefill and a decode step, and a whole decode
    step (append + attend) eager and replayed from a captured graph."""
    res = {}
    steps, warm = max(5, min(args.steps, 20)), max(1, args.warmup)

    def decode_line(name, b):
        db = device.to_device(b, plan="balanced")
        ms = _time_calls(torch, lambda i: device.run(db), steps, warm)
        gbs = kv_bytes_of(b) / (ms * 1e-3) / 1e9
        alg = decode_algorithmic_bytes(b) / (ms * 1e-3) / 1e9
        res[name] = dict(workload=b.name, call="sink_attn_decode (automatic plan: balanced)",
                         ms_per_call=round(ms, 5), kv_gbs=round(gbs, 1),
                         frac_hbm=round(alg / HBM_PEAK_GBS, 4))
        del db
        torch.cuda.empty_cache()

    def prefill_line(name, b, call="sink_attn_prefill"):
        db = device.to_device(b, with_lse=False)
        ms = _time_calls(torch, lambda i: device.run(db), steps, warm)
        flops = prefill_pairs(b) * 4 * b.head_dim
        tfs = flops / (ms * 1e-3) / 1e12
        res[name] = dict(workload=b.name, call=call, ms_per_call=round(ms, 5),
                         tflops=round(tfs, 2), frac_mfma=round(tfs / BF16_PEAK_TFLOPS, 4),
                         kv_gbs=round(kv_bytes_of(b) / (ms * 1e-3) / 1e9, 1))
        del db
        torch.cuda.empty_cache()

    log("[bench] extra: workload 3")
    decode_line("c3_split_decode", W.config(3))
    log("[bench] extra: workload 5")
    mx = W.config(5)
    prefill_line("c5_prefill", mx.prefill)
    decode_line("c5_decode", mx.decode)
    del mx
    log("[bench] extra: verification batch")
    vb = W.verify_workload("verify_4tok")
    prefill_line("verify_4tok_prefill", vb, call="sink_attn_prefill (qlen 4 per request)")

    def verify_line(name, b, call):
        db = device.to_device(b, with_lse=False, plan="verify")
        ms = _time_calls(torch, lambda i: device.run(db), steps, warm)
        # reads as a decode, plus the output rows written (fp32)
        alg = decode_algorithmic_bytes(b) + b.total_q * b.num_qo_heads * b.head_dim * 4
        res[name] = dict(
            workload=b.name, call=call, ms_per_call=round(ms, 5),
            kv_gbs=round(kv_bytes_of(b) / (ms * 1e-3) / 1e9, 1),
            frac_hbm=round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        del db
        torch.cuda.empty_cache()

    verify_line("verify_4tok", vb, "sink_attn_verify (automatic split plan)")
    log("[bench] extra: tree verification batch")
    verify_line("verify_16tok_causal", W.verify_workload("verify_16tok"),
                "sink_attn_verify (linear 16-token drafts, causal; 128-row tiles)")
    verify_line("verify_tree_16tok", W.verify_workload("verify_tree_16tok"),
                "sink_attn_verify_tree (one mask word per token; 128-row tiles)")
    verify_line("verify_tree_32tok", W.verify_workload("verify_tree_32tok"),
                "sink_attn_verify_tree (automatic plan: 128-row tiles)")
    log("[bench] extra: bias + rotary + paged append")
    append_lines(args, torch, sa, W, res, steps, warm)
    log("[bench] extra: decode step, eager and as a captured graph")
    graph_step_line(torch, sa, W, res, steps, warm)
    return res


def graph_step_line(torch, sa, W, res, steps, warm):
    """One decode step of 64 requests (64q/8kv, KV lengths U[1, 4096]): the
    new token's bias + rotary + paged append, then the automatic-plan decode
    (balanced first pass + finish), launched eagerly and replayed from one
    captured HIP graph.  Whole step per call, HIP events."""
    B, Hq, Hkv = 64, 64, 8
    rng = np.random.default_rng(1095)
    L = rng.integers(1, 4097, size=B)
    ab = W.make_append_batch(rng, qlens=[1] * B, kv_lens=L, hq=Hq, hkv=Hkv, spare_pages=0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    qkv, bias, kp, vp = dev(ab.qkv), dev(ab.bias), dev(ab.k_pages), dev(ab.v_pages)
    qo, kl, pi, px = i32(ab.qo_indptr), i32(ab.kv_len), i32(ab.page_indptr), i32(ab.page_indices)
    table = torch.empty((4096, 64), dtype=torch.float32, device="cuda")
    sa.sink_attn_rope_table(table, 4096, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    sinks = torch.from_numpy(rng.standard_normal(Hq).astype(np.float32)).cuda()
    q = torch.empty((B, Hq, 64), dtype=torch.int16, device="cuda")
    out = torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    max_L = int(L.max())
    ws_bytes = sa.sink_attn_decode_workspace_size(B, Hq, Hkv, 64, max_L, 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    def call(i=0):
        sa.sink_attn_qkv_rope_append(qkv, bias, table, 4096, qo, kl, pi, px, B, Hq, Hkv, 64, 16,
                                     B, 0, q, kp, vp)
        sa.sink_attn_decode(q, kp, vp, pi, px, kl, sinks, B, Hq, Hkv, 64, 16, max_L, 0, 0.125, out,
                            sa.F32, lse, ws, ws_bytes)

    eager = _time_calls(torch, call, steps, warm)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    replay = _time_calls(torch, lambda i: graph.replay(), steps, warm)
    kv = int(L.sum()) * 2 * Hkv * 64 * 2
    res["decode_step_graph"] = dict(
        workload=f"decode step: B={B}, L~U[1,4096], 64q/8kv; append + attend",
        call="sink_attn_qkv_rope_append + sink_attn_decode (balanced), 3 kernels",
        ms_eager=round(eager, 5), ms_graph_replay=round(replay, 5),
        kv_gbs_graph=round(kv / (replay * 1e-3) / 1e9, 1))
    del graph


def append_lines(args, torch, sa, W, res, steps, warm):
    """sink_attn_qkv_rope_append on a prefill step (8 x 4096 new tokens, the
    causal-prefill shape) and a decode step (64 requests x 1 token), 64q/8kv,
    YaRN table of 131072 positions.  Algorithmic bytes: the qkv rows read and
    the q / k / v rows written (2 x T x (Hq + 2 Hkv) x 128 B), the table row of
    each token (256 B), the bias and the index arrays."""
    table = torch.empty((131072, 64), dtype=torch.float32, device="cuda")
    sa.sink_attn_rope_table(table, 131072, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    for name in W.APPEND_WORKLOADS:
        ab = W.append_workload(name)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
        qkv, bias, kp, vp = dev(ab.qkv), dev(ab.bias), dev(ab.k_pages), dev(ab.v_pages)
        qo, kl, pi, px = i32(ab.qo_indptr), i32(ab.kv_len), i32(ab.page_indptr), i32(ab.page_indices)
        q_out = torch.empty((ab.total_q, 64, 64), dtype=torch.int16, device="cuda")

        def call(i):
            sa.sink_attn_qkv_rope_append(qkv, bias, table, 131072, qo, kl, pi, px, ab.batch, 64, 8,
                                         64, 16, ab.total_q, 0, q_out, kp, vp)
        ms = _time_calls(torch, call, steps, warm)
        H = 64 + 2 * 8
        alg = (2 * ab.total_q * H * 128 + ab.total_q * 256 + H * 128
               + 4 * (2 * (ab.batch + 1) + ab.batch + len(ab.page_indices)))
        res[name] = dict(workload=f"{ab.total_q} new tokens, 64q/8kv, d=64, page 16, YaRN table",
                         call="sink_attn_qkv_rope_append", ms_per_call=round(ms, 5),
                         achieved_gbs=round(alg / (ms * 1e-3) / 1e9, 1),
                         frac_hbm=round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         algorithmic_bytes=int(alg))
        del qkv, bias, kp, vp, q_out
        torch.cuda.empty_cache()


def bench_prefill(args, torch, sa, device, W):
    b = W.config(4)
    db = device.to_device(b, with_lse=False)
    torch.cuda.synchronize()
    steps = max(5, min(args.steps, 20))
    for _ in range(max(1, args.warmup)):
        device.run(db)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        device.run(db)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(c) for a, c in evs]))
    flops = prefill_pairs(b) * 4 * b.head_dim
    tfs = flops / (ms * 1e-3) / 1e12
    return dict(workload=W.CONFIG_NAMES[4], value=round(tfs, 2), unit="TFLOP/s",
                ms_per_call=round(ms, 4), flop_per_call=flops, steps=steps,
                roofline=dict(bound="mfma", achieved=round(tfs, 2), peak=BF16_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(tfs / BF16_PEAK_TFLOPS, 4),
                              traffic=PREFILL_TRAFFIC_BYTES))


def cpu_baseline(b, kv_bytes, seconds):
    import oracle
    threads = len(os.sched_getaffinity(0))
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t = time.perf_counter()
        oracle.attend(b, nthreads=threads)
        times.append(time.perf_counter() - t)
        if time.perf_counter() >= t_end or len(times) >= 1000:
            break
    mean = float(np.mean(times))
    return dict(value=round(kv_bytes / mean / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                sample=f"the whole decode batch (64 requests, {int(b.kv_len.sum())} KV tokens, "
                       f"all 64 heads), fp64, {len(times)} run(s), mean {mean:.3f} s")


def traffic_run(torch, sa, device, W):
    """Untimed dispatches for hardware-counter passes (see module doc)."""
    x = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[traffic] copy: {x.numel() * 4} bytes read and written per dispatch")
    b = W.config(2)
    db = device.to_device(b, plan="balanced")
    B, Hq, D = db.batch, db.num_qo_heads, db.head_dim
    out_code = sa.F32 if db.out.dtype == torch.float32 else sa.BF16
    ks = [db.k] + [db.k.clone() for _ in range(KV_COPIES - 1)]
    vs = [db.v] + [db.v.clone() for _ in range(KV_COPIES - 1)]
    for i in range(8):
        sa.sink_attn_decode_balanced_partial(
            db.q, ks[i % KV_COPIES], vs[i % KV_COPIES], db.kv_indptr, db.page_indices, db.kv_len,
            db.sinks, B, Hq, db.num_kv_heads, D, db.page_size, db.max_kv_len, 0, db.sm_scale,
            db.out, out_code, db.lse, db.workspace, db.workspace_bytes)
    torch.cuda.synchronize()
    log(f"[traffic] decode first pass: {decode_algorithmic_bytes(b)} algorithmic bytes per dispatch")
    pb = W.config(4)
    pdb = device.to_device(pb, with_lse=False)
    for _ in range(3):
        device.run(pdb)
    torch.cuda.synchronize()
    log(f"[traffic] prefill: {prefill_pairs(pb) * 4 * pb.head_dim} flop per dispatch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--extra", action="store_true",
                    help="also time workloads 3 and 5 and a verification batch (adds ~2 min)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--mode", choices=["bench", "traffic"], default="bench")
    ap.add_argument("--decode-plan", choices=["balanced", "chunked"], default="balanced",
                    help="decode kernels to time (default: the automatic plan's, balanced)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus "
              f"{args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")

    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    import gqa_attention_sinks_attn_amd as sa
    from gqa_attention_sinks_attn_amd import device
    import workloads as W

    if args.mode == "traffic":
        traffic_run(torch, sa, device, W)
        return

    log("[bench] decode workload: generating inputs")
    dec = bench_decode(args, torch, sa, device, W)
    log(f"[bench] decode: {dec['ms_step']:.4f} ms/step, kernel {dec['kern_ms']:.4f} ms")
    pre = None
    if not args.no_prefill:
        log("[bench] prefill workload: generating inputs")
        pre = bench_prefill(args, torch, sa, device, W)
        log(f"[bench] prefill: {pre['ms_per_call']} ms, {pre['value']} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(dec["batch"], dec["kv_bytes"], args.cpu_seconds)

    b = dec["batch"]
    achieved = dec["alg_bytes"] / (dec["kern_ms"] * 1e-3) / 1e9
    line = {
        "metric": "sink-GQA prefill TFLOP/s and decode KV GB/s at 1 MI355X, % of roofline",
        "value": round(dec["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": W.CONFIG_NAMES[2],
            "batch": b.batch, "kv_tokens": int(b.kv_len.sum()), "num_qo_heads": b.num_qo_heads,
            "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "page_size": b.page_size,
            **dec["plan"], "kv_copies_rotated": KV_COPIES, "out_dtype": "f32",
            "step": ("sink_attn_decode_balanced_partial + sink_attn_decode_balanced_finish"
                     if args.decode_plan == "balanced"
                     else "sink_attn_decode_partial + sink_attn_merge"),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": DECODE_TRAFFIC_BYTES if args.decode_plan == "balanced" else None,
            "kernel": ("decode_balanced_kernel<8> (first pass)" if args.decode_plan == "balanced"
                       else "decode_kernel<8> (split-KV partial)"),
            "kernel_ms": round(dec["kern_ms"], 5), "kernel_samples": dec["kern_samples"],
            "algorithmic_bytes": dec["alg_bytes"],
        },
        "cpu_baseline": cpu,
    }
    if pre is not None:
        line["prefill"] = pre
    if args.extra:
        line["extra"] = bench_extra(args, torch, sa, device, W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
