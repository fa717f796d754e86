#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

Headline workload (the JSON line's `value`): paged decode, batch 64, KV
lengths uniform in [1, 4096], 64 query / 8 KV heads, head_dim 64, 16-token
pages with a permuted page table.  One step = one pass of the decode path
the library's automatic plan takes for it: the load-balanced first pass
(sink_attn_decode_balanced_partial, every wave streaming an equal share of
the batch's pages) followed by its finish pass (sink_attn_decode_balanced_
finish, the LSE merge of requests that span several ranges), both through
the C ABI.  `value` = KV bytes read per second (2 * Hkv * 64 * 2 B per KV
token) over the whole step.  --decode-plan chunked times the split-KV pair
(sink_attn_decode_partial + sink_attn_merge) instead.

Also on the same JSON line, every one on the same seeded inputs the parity
tests use:
  * "roofline": the headline step's dominant kernel (the first pass):
    algorithmic bytes per launch / its mean launch time from HIP events on
    the stream it runs on (every fourth launch of the timed region), against
    the 8 TB/s HBM peak;
  * "prefill": the causal prefill workload (8 x 4096 tokens, 64/8 heads,
    contiguous KV) in TFLOP/s against the 2.5 PFLOP/s dense bf16 peak;
  * "workloads": the long split-KV decode (4 x 131,072 keys, 32 chunks
    merged by LSE, sinks of standard deviation 2) and the two calls of the
    mixed ragged batch (16 chunked prefills on cached prefixes, then 256
    decodes), each with its own roofline, plus the two mixed calls back to
    back on one stream;
  * "cpu_baseline": the fp64 oracle timed on this host's cores: the whole
    decode batch (repeated), a bounded block of the causal prefill, the tiny
    prefill, single-thread times and the CPU model.

`traffic` (HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
passes over `--mode traffic`, each scaled by the same counter on a 256 MiB
copy) is reported only while the kernel sources hash to the values the
counters were taken on; otherwise null.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --mode traffic   # kernels only, for rocprofv3 --pmc passes
    python bench.py --mode shapes    # the prefill kernel at three sequence lengths, for --pmc
"""
from __future__ import annotations

import argparse
import hashlib
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
BURST = 32                     # back-to-back first-pass launches timed as one block
CSRC = os.path.join(ROOT, "gqa_attention_sinks_attn_amd", "csrc")

# HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, scaled by the 256 MiB
# copy's counters; profiles/ holds the summaries and commands), keyed by the
# kernel and by the hash of the sources that build it.  A source change
# makes the figure stale: it is then reported as null until retaken.
TRAFFIC = {
    "c2": (260_939_419, "decode_balanced.hip", "eeea2d547a1c646c"),
    "c3": (1_076_439_260, "decode_balanced.hip", "eeea2d547a1c646c"),
    "c4": (1_107_493_841, "prefill.hip", "c3f96a6225b93810"),
    "c5_prefill": (1_066_478_760, "prefill.hip", "c3f96a6225b93810"),
    "c5_decode": (4_355_381_223, "decode_balanced.hip", "eeea2d547a1c646c"),
}


def sources_hash(main: str) -> str:
    """The kernel's own source and the device helpers it includes."""
    h = hashlib.sha256()
    for f in (main, "common.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_of(workload: str):
    nbytes, main, digest = TRAFFIC[workload]
    if nbytes is None or sources_hash(main) != digest:
        return None
    return nbytes


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def decode_algorithmic_bytes(b, out_elem_bytes: int = 4) -> int:
    """Bytes the definition reads and writes once: K and V of every KV token
    (2 * Hkv * D * 2 B each), the queries, the output rows and their LSE,
    page ids, per-request lengths and page offsets, and the sinks."""
    L = b.kv_len.astype(np.int64)
    kv = int(L.sum()) * 2 * b.num_kv_heads * b.head_dim * 2
    rows = int(b.qo_indptr[-1]) * b.num_qo_heads
    q = rows * b.head_dim * 2
    out = rows * b.head_dim * out_elem_bytes + rows * 4
    pages = int(((L + b.page_size - 1) // b.page_size).sum()) * 4
    sinks = b.num_qo_heads * 4 if b.sinks is not None else 0
    return kv + q + out + pages + b.batch * 4 + (b.batch + 1) * 4 + sinks


def kv_bytes_of(b) -> int:
    return int(b.kv_len.astype(np.int64).sum()) * 2 * b.num_kv_heads * b.head_dim * 2


def prefill_pairs(b) -> int:
    """Unmasked (query row, head, key) triples of a prefill (causal or not)."""
    qlens = np.diff(b.qo_indptr).astype(np.int64)
    kvl = b.kv_len.astype(np.int64)
    if not b.causal:
        return int((qlens * kvl).sum()) * b.num_qo_heads
    # query t sees keys 0 .. kv_len - qlen + t  ->  sum_t (kv_len - qlen + t + 1)
    per_req = qlens * (kvl - qlens) + qlens * (qlens + 1) // 2
    return int(per_req.sum()) * b.num_qo_heads


def prefill_flops(b) -> int:
    return prefill_pairs(b) * 4 * b.head_dim


# ------------------------------------------------------------------ decode

def time_decode(torch, sa, device, b, steps, warmup, balanced=True, kv_copies=1,
                event_every=1, burst=BURST):
    """Times the decode of batch b: the whole step (first pass + finish,
    events around the timed region of `steps` steps) and the first pass:
    events around a block of `burst` back-to-back first-pass launches on the
    rotated KV copies, right after the steps (the kernel's average launch
    duration, as a kernel trace reports it), and, for reference, events
    around every `event_every`-th launch inside the steps (each such pair
    adds the event packets' own few microseconds to a ~50 us launch)."""
    db = device.to_device(b, plan="balanced" if balanced else "chunked")
    B, Hq, D = db.batch, db.num_qo_heads, db.head_dim
    out_code = sa.F32 if db.out.dtype == torch.float32 else sa.BF16
    if balanced:
        plan = dict(num_ranges=sa.sink_attn_decode_num_ranges(B, db.num_kv_heads,
                                                               db.max_kv_len, 0))
    else:
        S = device.splits_of(db)
        o_parts = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
        lse_parts = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        plan = dict(num_splits=S)
    ks = [db.k] + [db.k.clone() for _ in range(kv_copies - 1)]
    vs = [db.v] + [db.v.clone() for _ in range(kv_copies - 1)]
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
        k, v = ks[i % kv_copies], vs[i % kv_copies]
        if ev is not None:
            ev[0].record()
        first(k, v)
        if ev is not None:
            ev[1].record()
        second()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Each pair of event records costs the stream a few microseconds, so on
    # a short kernel only every event_every-th step is bracketed.
    sampled = [i for i in range(steps) if i % event_every == 0]
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in sampled}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i, evs.get(i))
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    single_ms = float(np.mean([a.elapsed_time(c) for a, c in evs.values()]))
    kern_ms = single_ms
    if burst > 0:
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record()
        for i in range(burst):
            first(ks[(steps + i) % kv_copies], vs[(steps + i) % kv_copies])
        b1.record()
        second()   # leave the outputs of a whole step behind
        torch.cuda.synchronize()
        kern_ms = b0.elapsed_time(b1) / burst
    res = dict(db=db, plan=plan, ms_step=ms_step, kern_ms=kern_ms,
               kern_samples=burst if burst > 0 else len(evs),
               kern_single_ms=single_ms, kern_single_samples=len(evs),
               kv_bytes=kv_bytes_of(b), alg_bytes=decode_algorithmic_bytes(b),
               first=first, ks=ks, vs=vs)
    return res


def decode_entry(name, b, r, kernel, traffic=None):
    """JSON object of one timed decode workload."""
    achieved = r["alg_bytes"] / (r["kern_ms"] * 1e-3) / 1e9
    whole = r["alg_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    return {
        "workload": name, **r["plan"],
        "call": "sink_attn_decode_balanced_partial + sink_attn_decode_balanced_finish "
                "(the automatic plan of sink_attn_decode)",
        "ms_per_call": round(r["ms_step"], 5),
        "kv_gbs": round(r["kv_bytes"] / (r["ms_step"] * 1e-3) / 1e9, 1),
        "whole_call_frac_hbm": round(whole / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kernel, "kernel_ms": round(r["kern_ms"], 5),
            "kernel_samples": r["kern_samples"],
            "kernel_timing": f"HIP events around {r['kern_samples']} back-to-back first-pass "
                             "launches on rotated KV copies (cache-cold), after the timed steps",
            "kernel_ms_single_brackets": round(r["kern_single_ms"], 5),
            "algorithmic_bytes": r["alg_bytes"],
        },
    }


# ----------------------------------------------------------------- prefill

def time_prefill(torch, device, b, steps, warmup):
    db = device.to_device(b, with_lse=False)
    torch.cuda.synchronize()
    for _ in range(max(1, warmup)):
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
    return db, ms


def prefill_entry(name, b, ms, steps, traffic=None):
    flops = prefill_flops(b)
    tfs = flops / (ms * 1e-3) / 1e12
    return dict(workload=name, call="sink_attn_prefill", value=round(tfs, 2), unit="TFLOP/s",
                ms_per_call=round(ms, 4), flop_per_call=flops, steps=steps,
                roofline=dict(bound="mfma", achieved=round(tfs, 2), peak=BF16_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(tfs / BF16_PEAK_TFLOPS, 4),
                              traffic=traffic, kernel=f"prefill_kernel<{b.num_qo_heads // b.num_kv_heads}, "
                                                      f"{'true' if b.page_indices is not None else 'false'}, false>"))


def bench_workloads(args, torch, sa, device, W):
    """Workloads 3 and 5, each with its own roofline."""
    out = {}
    steps = max(5, min(args.steps, 20))
    warm = max(1, args.warmup)
    log("[bench] workload 3: long split-KV decode")
    b3 = W.config(3)
    r3 = time_decode(torch, sa, device, b3, steps, warm)
    out["c3_split_decode"] = decode_entry(W.CONFIG_NAMES[3], b3, r3,
                                          "decode_balanced_kernel<8, false> (first pass)",
                                          traffic=traffic_of("c3"))
    out["c3_split_decode"]["note"] = (
        "the 32 chunks of the workload are the page ranges of the automatic plan; "
        "the split-KV pair with S = 32 is timed under extra")
    del r3
    torch.cuda.empty_cache()

    log("[bench] workload 5: mixed ragged batch")
    mx = W.config(5)
    pdb, pms = time_prefill(torch, device, mx.prefill, steps, warm)
    out["c5_prefill"] = prefill_entry(W.CONFIG_NAMES[5] + " -- (i) chunked prefills",
                                      mx.prefill, pms, steps, traffic=traffic_of("c5_prefill"))
    r5 = time_decode(torch, sa, device, mx.decode, steps, warm)
    out["c5_decode"] = decode_entry(W.CONFIG_NAMES[5] + " -- (ii) decodes", mx.decode, r5,
                                    "decode_balanced_kernel<8, false> (first pass)",
                                    traffic=traffic_of("c5_decode"))
    # both calls back to back on one stream, as one step of the mixed batch
    ddb = r5["db"]

    def both(i):
        device.run(pdb)
        device.run(ddb)
    seq_ms = _time_calls(torch, both, steps, warm)
    flops = prefill_flops(mx.prefill)
    kvb = kv_bytes_of(mx.decode)
    out["c5_sequential"] = dict(
        call="sink_attn_prefill then sink_attn_decode (automatic plan), one stream",
        ms_per_step=round(seq_ms, 4),
        sum_of_calls_ms=round(pms + r5["ms_step"], 4),
        prefill_tflops_share=round(flops / (seq_ms * 1e-3) / 1e12, 2),
        decode_kv_gbs_share=round(kvb / (seq_ms * 1e-3) / 1e9, 1))
    del pdb, r5, ddb, mx
    torch.cuda.empty_cache()
    return out


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


# -------------------------------------------------------------- CPU oracle

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, dec_batch, seconds):
    """The oracle as it stands (fp64, OpenMP over (row, head)), timed on this
    host: the whole decode batch repeated for about `seconds`; a contiguous
    block of causal-prefill rows (all heads) sized to about `seconds`; the
    tiny prefill (mean of 10); single-thread times of the tiny prefill and
    the decode batch; the long split decode once."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    steady = time.perf_counter

    def timed(fn):
        t = steady()
        fn()
        return steady() - t

    # decode (the headline workload), whole batch, repeated
    times = []
    t_end = steady() + seconds
    while True:
        times.append(timed(lambda: oracle.attend(dec_batch, nthreads=threads)))
        if steady() >= t_end or len(times) >= 1000:
            break
    dec_mean = float(np.mean(times))
    kvb = kv_bytes_of(dec_batch)
    L = dec_batch.kv_len.astype(np.int64)
    dec_flops = int(L.sum()) * dec_batch.num_qo_heads * 4 * dec_batch.head_dim

    # prefill: rows of one request of the causal prefill workload, all heads,
    # in row order (the oracle's own traversal), from its last row backwards
    # until the block holds about `seconds` of work at a probed rate
    b4 = W.config(4)
    qlen = int(b4.qo_indptr[1] - b4.qo_indptr[0])
    probe_rows = 64
    rows = np.repeat(np.arange(qlen - probe_rows, qlen, dtype=np.int64), b4.num_qo_heads)
    heads = np.tile(np.arange(b4.num_qo_heads, dtype=np.int32), probe_rows)
    t_probe = timed(lambda: oracle.attend_rows(b4, rows, heads, nthreads=threads))
    n_rows = int(min(qlen, max(probe_rows, probe_rows * seconds / max(t_probe, 1e-3))))
    r0 = qlen - n_rows
    rows = np.repeat(np.arange(r0, qlen, dtype=np.int64), b4.num_qo_heads)
    heads = np.tile(np.arange(b4.num_qo_heads, dtype=np.int32), n_rows)
    t_pre = timed(lambda: oracle.attend_rows(b4, rows, heads, nthreads=threads))
    # query t of a 4096-token request sees t + 1 keys
    pre_flops = int(np.arange(r0 + 1, qlen + 1, dtype=np.int64).sum()) * b4.num_qo_heads \
        * 4 * b4.head_dim
    pre_rate = pre_flops / t_pre
    c4_flops = prefill_flops(b4)
    del b4

    b1 = W.config(1)
    c1_flops = prefill_flops(b1)
    c1_mean = float(np.mean([timed(lambda: oracle.attend(b1, nthreads=threads))
                             for _ in range(10)]))
    c1_single = float(np.mean([timed(lambda: oracle.attend(b1, nthreads=1)) for _ in range(10)]))
    c2_single = timed(lambda: oracle.attend(dec_batch, nthreads=1))

    b3 = W.config(3)
    c3_s = timed(lambda: oracle.attend(b3, nthreads=threads))
    c3_flops = int(b3.kv_len.astype(np.int64).sum()) * b3.num_qo_heads * 4 * b3.head_dim
    del b3

    return dict(
        value=round(kvb / dec_mean / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
        sample=f"the whole decode batch (64 requests, {int(L.sum())} KV tokens, all 64 heads), "
               f"fp64, {len(times)} run(s), mean {dec_mean:.3f} s",
        cpu_model=cpu_model(),
        prefill=dict(
            value=round(pre_rate / 1e9, 3), unit="GFLOP/s", cores=threads, kind="oracle",
            sample=f"causal prefill 8 x 4096, 64q/8kv: rows {r0}..{qlen - 1} of request 0, all "
                   f"64 heads ({pre_flops / 1e9:.1f} GFLOP) in {t_pre:.2f} s",
            whole_workload_s_at_this_rate=round(c4_flops / pre_rate, 1)),
        per_workload=dict(
            c1_s=round(c1_mean, 5), c1_gflops=round(c1_flops / c1_mean / 1e9, 3),
            c2_s=round(dec_mean, 4), c2_gflops=round(dec_flops / dec_mean / 1e9, 3),
            c3_s=round(c3_s, 3), c3_gflops=round(c3_flops / c3_s / 1e9, 3)),
        single_thread=dict(c1_s=round(c1_single, 5), c2_s=round(c2_single, 3)),
    )


# ------------------------------------------------------------------ extras

def bench_extra(args, torch, sa, device, W):
    """Other batches, each timed whole (all kernels of the call), HIP events:
    the split-KV pair on the long decode, a multi-token verification batch
    (64 requests, 4 drafted tokens each, KV lengths U[4, 4096]) through
    sink_attn_prefill and sink_attn_verify, and 16-token drafts (linear,
    then random trees) through sink_attn_verify and sink_attn_verify_tree,
    the bias + rotary + paged-append step on a prefill and a decode step,
    and a whole decode step (append + attend) eager and replayed from a
    captured graph."""
    res = {}
    steps, warm = max(5, min(args.steps, 20)), max(1, args.warmup)

    log("[bench] extra: workload 3 through the split-KV pair (32 chunks, then the merge)")
    b3 = W.config(3)
    db3 = device.to_device(b3, plan="chunked")
    ms = _time_calls(torch, lambda i: device.run(db3), steps, warm)
    res["c3_split_kv_pair"] = dict(workload=b3.name, call="sink_attn_decode (num_splits = 32)",
                                   ms_per_call=round(ms, 5),
                                   kv_gbs=round(kv_bytes_of(b3) / (ms * 1e-3) / 1e9, 1),
                                   frac_hbm=round(decode_algorithmic_bytes(b3) / (ms * 1e-3)
                                                  / 1e9 / HBM_PEAK_GBS, 4))
    del db3, b3
    torch.cuda.empty_cache()

    def prefill_line(name, b, call="sink_attn_prefill"):
        db = device.to_device(b, with_lse=False)
        ms = _time_calls(torch, lambda i: device.run(db), steps, warm)
        tfs = prefill_flops(b) / (ms * 1e-3) / 1e12
        res[name] = dict(workload=b.name, call=call, ms_per_call=round(ms, 5),
                         tflops=round(tfs, 2), frac_mfma=round(tfs / BF16_PEAK_TFLOPS, 4),
                         kv_gbs=round(kv_bytes_of(b) / (ms * 1e-3) / 1e9, 1))
        del db
        torch.cuda.empty_cache()

    log("[bench] extra: verification batch")
    vb = W.verify_workload("verify_4tok")
    prefill_line("verify_4tok_prefill", vb, call="sink_attn_prefill (qlen 4 per request)")

    def verify_line(name, b, call):
        db = device.to_device(b, with_lse=False, plan="verify")
        ms = _time_calls(torch, lambda i: device.run(db), steps, warm)
        # reads as a decode (the output rows fp32, no LSE)
        alg = decode_algorithmic_bytes(b) - b.total_q * b.num_qo_heads * 4
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

    def attend(i=0):
        sa.sink_attn_decode(q, kp, vp, pi, px, kl, sinks, B, Hq, Hkv, 64, 16, max_L, 0, 0.125, out,
                            sa.F32, lse, ws, ws_bytes)

    fws_bytes = sa.sink_attn_decode_step_workspace_size(B, Hq, Hkv, 64, max_L)
    fws = torch.empty(max(fws_bytes, 256), dtype=torch.uint8, device="cuda")

    def fused(i=0):
        sa.sink_attn_decode_step(qkv, bias, table, 4096, 0, kp, vp, pi, px, kl, sinks, B, Hq, Hkv,
                                 64, 16, max_L, 0.125, out, sa.F32, lse, fws, fws_bytes)

    def replayed(fn):
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn()
        torch.cuda.synchronize()
        ms = _time_calls(torch, lambda i: graph.replay(), steps, warm)
        del graph
        return ms

    eager = _time_calls(torch, call, steps, warm)
    attend_only = _time_calls(torch, attend, steps, warm)
    fused_eager = _time_calls(torch, fused, steps, warm)
    replay = replayed(call)
    fused_replay = replayed(fused)
    kv = int(L.sum()) * 2 * Hkv * 64 * 2
    res["decode_step_graph"] = dict(
        workload=f"decode step: B={B}, L~U[1,4096], 64q/8kv; append + attend",
        call="sink_attn_qkv_rope_append + sink_attn_decode (balanced), 3 kernels",
        ms_eager=round(eager, 5), ms_attend_only=round(attend_only, 5),
        ms_graph_replay=round(replay, 5),
        kv_gbs_graph=round(kv / (replay * 1e-3) / 1e9, 1))
    res["decode_step_fused"] = dict(
        workload=f"decode step: B={B}, L~U[1,4096], 64q/8kv; append + attend",
        call="sink_attn_decode_step (the append inside the balanced first pass), 2 kernels",
        ms_eager=round(fused_eager, 5), ms_graph_replay=round(fused_replay, 5),
        kv_gbs=round(kv / (fused_eager * 1e-3) / 1e9, 1))


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
        if name == "append_prefill_8x4096":
            # the whole prefill step: append then attend, against the fused call
            qlens = np.diff(ab.qo_indptr)
            max_qlen, max_L = int(qlens.max()), int(ab.kv_len.max())
            sinks = torch.from_numpy(
                np.random.default_rng(1096).standard_normal(64).astype(np.float32)).cuda()
            out = torch.empty((ab.total_q, 64, 64), dtype=torch.float32, device="cuda")
            lse = torch.empty((ab.total_q, 64), dtype=torch.float32, device="cuda")

            def pair(i):
                call(i)
                sa.sink_attn_prefill(q_out, qo, kp, vp, pi, px, kl, sinks, ab.batch, 64, 8, 64, 16,
                                     ab.total_q, max_qlen, max_L, 0.125, 1, out, sa.F32, lse)

            def fused(i):
                sa.sink_attn_prefill_step(qkv, bias, table, 131072, 0, qo, kp, vp, pi, px, kl,
                                          sinks, ab.batch, 64, 8, 64, 16, ab.total_q, max_qlen,
                                          max_L, 0.125, 1, out, sa.F32, lse)
            ms_pair = _time_calls(torch, pair, steps, warm)
            ms_fused = _time_calls(torch, fused, steps, warm)
            flops = sum(int(q) * (2 * int(L) - int(q) + 1) // 2 for q, L in zip(qlens, ab.kv_len)) \
                * 64 * 4 * 64
            res["prefill_step_8x4096"] = dict(
                workload=f"prefill step: {ab.total_q} new tokens, 64q/8kv, d=64, page 16, YaRN",
                call="sink_attn_qkv_rope_append + sink_attn_prefill, against sink_attn_prefill_step",
                ms_pair=round(ms_pair, 5), ms_fused=round(ms_fused, 5),
                tflops_fused=round(flops / (ms_fused * 1e-3) / 1e12, 2))
            del out, lse
        del qkv, bias, kp, vp, q_out
        torch.cuda.empty_cache()


# ----------------------------------------------------------------- traffic

def traffic_run(torch, sa, device, W):
    """Untimed dispatches for hardware-counter passes, in this order: a plain
    256 MiB device-to-device copy three times (the calibration dispatch for
    FETCH_SIZE / WRITE_SIZE), the headline decode's first pass eight times
    (rotating the same four KV copies as the timed run), the causal prefill
    three times, the long split decode's first pass three times, the mixed
    batch's prefill and decode first pass three times each, then the
    16-token verification batch and the 32-token draft trees three times
    each."""
    x = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[traffic] copy: {x.numel() * 4} bytes read and written per dispatch")
    del x, y
    b = W.config(2)
    r = time_decode(torch, sa, device, b, steps=8, warmup=0, kv_copies=KV_COPIES, burst=0)
    log(f"[traffic] decode first pass x8: {decode_algorithmic_bytes(b)} algorithmic bytes")
    del r
    pb = W.config(4)
    pdb = device.to_device(pb, with_lse=False)
    for _ in range(3):
        device.run(pdb)
    torch.cuda.synchronize()
    log(f"[traffic] prefill x3: {prefill_flops(pb)} flop per dispatch")
    del pdb, pb
    b3 = W.config(3)
    r = time_decode(torch, sa, device, b3, steps=3, warmup=0, burst=0)
    log(f"[traffic] long decode first pass x3: {decode_algorithmic_bytes(b3)} algorithmic bytes")
    del r, b3
    mx = W.config(5)
    pdb = device.to_device(mx.prefill, with_lse=False)
    for _ in range(3):
        device.run(pdb)
    torch.cuda.synchronize()
    log(f"[traffic] mixed prefill x3: {prefill_flops(mx.prefill)} flop per dispatch")
    r = time_decode(torch, sa, device, mx.decode, steps=3, warmup=0, burst=0)
    log(f"[traffic] mixed decode first pass x3: {decode_algorithmic_bytes(mx.decode)} "
        f"algorithmic bytes")
    torch.cuda.synchronize()
    del r, pdb, mx
    torch.cuda.empty_cache()
    for name in ("verify_16tok", "verify_tree_32tok"):
        vb = W.verify_workload(name)
        vdb = device.to_device(vb, plan="verify")
        for _ in range(3):
            device.run(vdb)
        torch.cuda.synchronize()
        log(f"[traffic] {name} x3: {kv_bytes_of(vb)} bytes of KV")
        del vdb, vb


def shapes_run(torch, device, W):
    """Untimed dispatches for counter passes on the prefill kernel across
    sequence lengths (64 q / 8 KV heads, contiguous cache, seed 7), two each,
    in this order: causal 8 x 4,096, causal 2 x 16,384, non-causal 8 x 4,096.
    The same number of workgroups (8,192) with 32.5, 128.5 and 64 key tiles
    each on average: the counters separate the per-tile cost from the
    per-workgroup one."""
    shapes = [("causal 8 x 4096", [4096] * 8, True), ("causal 2 x 16384", [16384] * 2, True),
              ("non-causal 8 x 4096", [4096] * 8, False)]
    for name, lens, causal in shapes:
        b = W.make_batch(7, kind="prefill", qlens=lens, kv_lens=lens, hq=64, hkv=8,
                         sinks="normal", paged=False, causal=causal)
        db = device.to_device(b, with_lse=False)
        torch.cuda.synchronize()
        for _ in range(2):
            device.run(db)
            torch.cuda.synchronize()
        log(f"[shapes] {name} x2: {prefill_flops(b)} flop per dispatch")
        del db, b
        torch.cuda.empty_cache()


# -------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true", help="skip the causal prefill")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the long decode and the mixed batch")
    ap.add_argument("--extra", action="store_true",
                    help="also time the split-KV pair, verification, append and graph batches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--mode", choices=["bench", "traffic", "shapes"], default="bench",
                    help="traffic / shapes: untimed dispatches for rocprofv3 counter passes")
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
    if args.mode == "shapes":
        shapes_run(torch, device, W)
        return

    log("[bench] decode workload: generating inputs")
    b = W.config(2)
    balanced = args.decode_plan == "balanced"
    dec = time_decode(torch, sa, device, b, args.steps, args.warmup, balanced=balanced,
                      kv_copies=KV_COPIES, event_every=EVENT_EVERY)
    log(f"[bench] decode: {dec['ms_step']:.4f} ms/step, first pass {dec['kern_ms']:.4f} ms")
    plan = dec["plan"]
    del dec["db"], dec["ks"], dec["vs"], dec["first"]
    torch.cuda.empty_cache()
    pre = None
    if not args.no_prefill:
        log("[bench] prefill workload: generating inputs")
        b4 = W.config(4)
        _, ms = time_prefill(torch, device, b4, max(5, min(args.steps, 20)), args.warmup)
        pre = prefill_entry(W.CONFIG_NAMES[4], b4, ms, max(5, min(args.steps, 20)),
                            traffic=traffic_of("c4"))
        log(f"[bench] prefill: {pre['ms_per_call']} ms, {pre['value']} TFLOP/s")
        del b4
        torch.cuda.empty_cache()
    wl = None
    if not args.no_workloads:
        wl = bench_workloads(args, torch, sa, device, W)
        for k, v in wl.items():
            if "roofline" in v:
                log(f"[bench] {k}: {v['ms_per_call']} ms, roofline frac {v['roofline']['frac']}")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(W, b, args.cpu_seconds)

    achieved = dec["alg_bytes"] / (dec["kern_ms"] * 1e-3) / 1e9
    whole = dec["alg_bytes"] / (dec["ms_step"] * 1e-3) / 1e9
    line = {
        "metric": "sink-GQA prefill TFLOP/s and decode KV GB/s at 1 MI355X, % of roofline",
        "value": round(dec["kv_bytes"] / (dec["ms_step"] * 1e-3) / 1e9, 2),
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
            **plan, "kv_copies_rotated": KV_COPIES, "out_dtype": "f32",
            "step": ("sink_attn_decode_balanced_partial + sink_attn_decode_balanced_finish"
                     if balanced else "sink_attn_decode_partial + sink_attn_merge"),
            "whole_step_frac_hbm": round(whole / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_of("c2") if balanced else None,
            "kernel": ("decode_balanced_kernel<8, false> (first pass)" if balanced
                       else "decode_kernel<8> (split-KV partial)"),
            "kernel_ms": round(dec["kern_ms"], 5), "kernel_samples": dec["kern_samples"],
            "kernel_timing": f"HIP events around {dec['kern_samples']} back-to-back first-pass "
                             f"launches on the {KV_COPIES} rotated KV copies, after the timed steps",
            "kernel_ms_single_brackets": round(dec["kern_single_ms"], 5),
            "algorithmic_bytes": dec["alg_bytes"],
        },
        "cpu_baseline": cpu,
    }
    if pre is not None:
        line["prefill"] = pre
    if wl is not None:
        line["workloads"] = wl
    if args.extra:
        line["extra"] = bench_extra(args, torch, sa, device, W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
