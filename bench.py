"""Benchmark of the paged GQA attention hot path on one MI355X.

One "step" is one full forward pass (all kernels of the path: split-KV decode
partials + log-sum-exp combine, or the prefill kernel) over one batch of
synthetic, seeded input already resident in HBM.

Default workload: the decode batch (64 sequences x 1 query token, 32 q / 8 KV
heads, head_dim 128, page 64, KV lengths uniform in [1024, 8192], causal),
reported as achieved HBM GB/s of algorithmic bytes (K and V read once per KV
head, plus Q and the output): W warmup steps, then K timed steps.  Secondary
lines (the tiny mixed call's latency, long-context decode on both pool
layouts, chunked prefill, DiT non-causal, the quantised DiT path, and
variants) follow, each after a time-bounded warmup.
Prefill lines are in TFLOP/s of algorithmic FLOPs (4 * D per visible
(query, q head, key) triple).  Every line carries its roofline block; the
primary line and the tiny, long-decode, chunked-prefill, DiT and quantised
lines carry the fp64 CPU oracle timed on a bounded sample of the same
workload.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, 2.5 PFLOP/s
Q8_PEAK_TOPS = 5000.0          # MI355X dense int8 / fp8 MFMA, 5.0 P(FL)OP/s
METRIC = "decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% bf16 MFMA peak)"

DESCR = {
    "decode_batch": "decode batch: 64 seqs x 1 query token, 32 q / 8 KV heads (GQA 4), head_dim 128, "
                    "page 64, KV lengths U[1024, 8192], shuffled shared page pool, causal",
    "long_decode": "long-context decode: 128 seqs x 1 token, 16 q / 2 KV heads (GQA 8), head_dim 256, "
                   "page 64, context 32768, 1% outlier K rows x4, causal",
    "chunked_prefill": "chunked prefill: 8 seqs, new tokens U[512, 4096] after cached context U[0, 8192], "
                       "24 q / 4 KV heads, head_dim 256, page 64, causal",
    "dit_self_attn": "DiT self-attention: 1 seq x 37810 tokens, 56 heads (MHA), head_dim 128, "
                     "non-causal, per-channel K offset N(0, 2)",
    "tiny_mixed": "tiny mixed: 2 seqs x 32 queries, 24 q / 4 KV heads, head_dim 256, 22-page pool, causal",
    "short_batch": "short multi-token runs: 256 seqs x U[2, 8] query tokens, 32 q / 4 KV heads (GQA 8), "
                   "head_dim 128, page 64, KV lengths U[1024, 8192], causal",
}
BOUND = {"decode_batch": "hbm", "long_decode": "hbm", "chunked_prefill": "mfma",
         "dit_self_attn": "mfma", "tiny_mixed": "hbm", "short_batch": "hbm"}


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def visible_pairs(case) -> int:
    """Sum over (sequence, query) of visible keys."""
    tot = 0
    for n, L in zip(case.q_lens, case.kv_lens):
        if not case.causal:
            tot += n * L
        else:
            for i in range(n):
                tot += max(0, min(L, L - n + i + 1))
    return tot


def algorithmic_bytes(case, window: int = 0) -> int:
    """K and V of every visible key once per KV head, Q read once, out written once.
    With a window only keys from row 0's window start on are needed; an fp8
    cache holds one byte per element."""
    d, hq, hkv = case.head_dim, case.num_q_heads, case.num_kv_heads
    keys = sum(L if window <= 0 else min(L, L - max(0, L - n - window + 1)) for n, L in zip(case.q_lens, case.kv_lens))
    kv = keys * hkv * 2 * d * case.kv.element_size()
    T = sum(case.q_lens)
    return kv + 2 * T * hq * d * 2


def algorithmic_flops(case) -> int:
    return 4 * case.head_dim * case.num_q_heads * visible_pairs(case)


def _time_steps(fn, steps):
    """Average ms per call of fn() over `steps` calls, events on the current stream."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def _step_distribution(fn, steps):
    """Per-step ms from an event pair around each call (a separate pass):
    mean, p50, p90, min, max."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda q: ts[min(len(ts) - 1, int(round(q * (len(ts) - 1))))]
    return {"mean": round(sum(ts) / len(ts), 4), "p50": round(pick(0.5), 4), "p90": round(pick(0.9), 4),
            "min": round(ts[0], 4), "max": round(ts[-1], 4)}


def stream_read_ceiling(nbytes, launches=50, configs=((256, 8), (512, 4), (512, 8), (1024, 4), (2048, 4))):
    """The on-box read ceiling: GB/s of the library's plain streaming-read
    kernel over a buffer of nbytes (best over a few grid sizes and load
    depths)."""
    import paged_kv_gqa_fwd_amd as pa
    n = (nbytes + 15) // 16 * 16
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(max(g for g, _ in configs) * 256, dtype=torch.int32, device="cuda")
    best = None
    for g, depth in configs:
        for _ in range(10):
            pa.stream_read(buf, g, sink, depth=depth)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(launches):
            pa.stream_read(buf, g, sink, depth=depth)
        t1.record()
        torch.cuda.synchronize()
        gbs = n / (t0.elapsed_time(t1) / launches * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, g, depth)
    del buf, sink
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 2), "grid": best[1], "loads_in_flight_per_thread": best[2], "bytes": n,
            "launches": launches}


def _kernel_times(fn, steps):
    """Per-kind average kernel ms from the library's per-launch HIP events
    (recorded on the launch stream), in a separate pass so the step timing
    above carries no instrumentation."""
    import paged_kv_gqa_fwd_amd as pa
    torch.cuda.synchronize()
    pa.kernel_timing_read()                      # discard anything recorded before
    pa.kernel_timing_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    pa.kernel_timing_enable(False)
    mm, mn, cm, cn, pm, pn, wm, wn = pa.kernel_timing_read()
    return mm / max(mn, 1), (cm / cn if cn else 0.0), (pm / pn if pn else 0.0), (wm / wn if wn else 0.0)


def _warm(fn, min_steps, min_seconds=0.3):
    """Untimed calls until at least min_steps were made and min_seconds of
    GPU time passed (the clocks settle only after a few hundred ms of load).
    Returns the mean ms per call of the last batch, an estimate for sizing
    the timed region."""
    done, t_start, per = 0, time.perf_counter(), None
    batch = max(1, min_steps)
    while True:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / batch * 1e3
        done += batch
        if done >= min_steps and time.perf_counter() - t_start >= min_seconds:
            return per
        batch = max(1, min(1000, int(0.1e3 / max(per, 1e-3))))


def _secondary_steps(per_ms, steps, seconds=0.4):
    """Timed steps of a secondary line: about `seconds` of work, at least 3,
    at most the primary line's K."""
    return max(3, min(steps, int(seconds * 1e3 / max(per_ms, 1e-3))))


def run_workload(name, steps, warmup, pps=0, path=0, window=0, fp8=False, layout=None, secondary=True, tag="",
                 case=None):
    """Time one workload: W warmup calls (time-bounded for secondary lines),
    then K timed calls; a second pass of calls with the library's per-launch
    events gives the kernel times, a third the per-step distribution.  `case`:
    inputs generated beforehand (else generated here)."""
    import paged_kv_gqa_fwd_amd as pa
    if case is None:
        log("[bench] generating %s%s%s%s" % (name, " (window %d)" % window if window else "",
                                           " (fp8 cache)" if fp8 else "", " (%s pool)" % layout if layout else ""))
        kw = {"layout": layout} if layout else {}
        case = workloads.WORKLOADS[name](device="cuda", **kw)
    kscale = 1.0
    if fp8:
        # e4m3 codes of 2x the bf16 pool values; scales 1/2 keep the values
        case = workloads.fp8_pool_case(case, mult=2.0)
        kscale = 0.5
    out = torch.empty_like(case.q)
    args = (case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, max(case.max_q, 1),
            case.scale, case.causal)
    dims = pa.make_dims(case.q, case.kv, case.block_table, out)
    plan = pa.make_plan(dims, case.n_seqs, max(case.max_q, 1), path, pps, window)

    def step():
        pa.paged_attention(*args, out=out, path=path, pages_per_split=pps, window=window, k_scale=kscale,
                           v_scale=kscale)

    if secondary:
        per = _warm(step, warmup)
        steps = _secondary_steps(per, steps)
    else:
        for _ in range(warmup):
            step()
    step_ms = _time_steps(step, steps)
    main_ms, comb_ms, _, _ = _kernel_times(step, steps)
    dist = _step_distribution(step, steps)
    suffix = ("+window%d" % window if window else "") + ("+fp8" if fp8 else "") + ("+%s" % layout if layout else "") + tag
    res = {
        "workload": name + suffix, "case": case, "steps": steps,
        "ms_per_step": step_ms, "step_ms_dist": dist,
        "main_kernel_ms": main_ms, "combine_kernel_ms": comb_ms,
        "path": {pa.PATH_SPLIT_DECODE: "split_decode+combine", pa.PATH_SPLIT_FUSED: "split_decode+merge",
                 pa.PATH_SPLIT_BALANCED: "balanced_split_decode+combine", pa.PATH_PREFILL: "prefill"}[plan.path],
        "pages_per_split": plan.pages_per_split, "max_splits": plan.max_splits,
        "bytes": algorithmic_bytes(case, window), "flops": algorithmic_flops(case),
    }
    return res


def run_write(name, steps, warmup):
    """The KV-cache write followed by attention in one call
    (attn_paged_fwd_write) on a workload's shape, with seeded new K/V rows
    for every query token.  On the split-decode paths the write runs inside
    the attention launch; the line also times the two-launch form (the write
    kernel, then attention) on the same inputs.  value = the step's
    algorithmic bytes (attention's, plus every new K/V byte read once and
    written once) per second."""
    import paged_kv_gqa_fwd_amd as pa
    log("[bench] generating %s (with KV-cache write)" % name)
    case = workloads.WORKLOADS[name](device="cuda")
    k_new, v_new = workloads.new_kv_tokens(case, case.seed + 1000)
    out = torch.empty_like(case.q)
    mq = max(case.max_q, 1)

    def step():
        pa.paged_attention_write(case.q, k_new, v_new, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                 mq, case.scale, case.causal, out=out)

    def two_launch():
        pa.kv_write(case.kv, k_new, v_new, case.block_table, case.seq_lens, case.cu_q, mq, q_like=case.q)
        pa.paged_attention(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, mq, case.scale,
                           case.causal, out=out)

    steps = _secondary_steps(_warm(step, warmup), steps)
    step_ms = _time_steps(step, steps)
    main_ms, comb_ms, _, write_ms = _kernel_times(step, steps)
    _warm(two_launch, warmup, 0.1)
    two_ms = _time_steps(two_launch, steps)
    _, _, _, write_alone_ms = _kernel_times(two_launch, steps)
    written = sum(min(n, L) for n, L in zip(case.q_lens, case.kv_lens))
    wbytes = 2 * written * case.num_kv_heads * 2 * case.head_dim * 2
    abytes = algorithmic_bytes(case)
    fused = write_ms == 0.0
    res = {"workload": name + "+kv_write", "value": round((abytes + wbytes) / (step_ms * 1e-3) / 1e9, 2),
           "unit": "GB/s (attention + write bytes)", "fused_write": fused, "write_bytes": wbytes,
           "ms_per_step": round(step_ms, 4), "steps": steps, "two_launch_ms_per_step": round(two_ms, 4),
           "gain_vs_two_launches": round(two_ms / step_ms - 1.0, 4),
           "write_kernel_ms_two_launch": round(write_alone_ms, 4),
           "write_kernel_GBps_two_launch": round(wbytes / (write_alone_ms * 1e-3) / 1e9, 2),
           "attention_ms": round(main_ms + comb_ms, 4), "path": "kv_write fused into attention" if fused else
           "kv_write kernel + attention"}
    kern_ms = main_ms if fused else write_ms
    if BOUND[name] == "hbm":
        ach = (abytes + wbytes if fused else wbytes) / (kern_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                           "kernel": "paged_decode_balanced_kernel (with the write)" if fused
                           else "paged_kv_write_kernel", "kernel_ms": round(kern_ms, 4)}
    else:
        ach = wbytes / (write_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "paged_kv_write_kernel",
                           "kernel_ms": round(write_ms, 4)}
    return res


def run_quant(steps, warmup, cpu_seconds=0.0):
    """The quantised path (attn_quant_fwd: preparation + fused int8/fp8 loop)
    on the video-DiT shape, same seeded Q/K/V as the bf16 DiT workload."""
    import paged_kv_gqa_fwd_amd as pa
    log("[bench] generating dit_self_attn (quantised path)")
    case = workloads.dit_self_attn(device="cuda")
    q, k, v = workloads.dense_from_case(case)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

    def step():
        pa.quant_attention(q, k, v, case.scale, False, out=out)

    steps = _secondary_steps(_warm(step, warmup), steps)
    step_ms = _time_steps(step, steps)
    main_ms, _, prep_ms, _ = _kernel_times(step, steps)
    dist = _step_distribution(step, steps)
    flops = algorithmic_flops(case)
    tops = flops / (step_ms * 1e-3) / 1e12
    loop_tops = flops / (main_ms * 1e-3) / 1e12
    res = {"workload": "dit_quant", "value": round(tops, 2),
           "unit": "TOPS (int8 Q.K ops + fp8 P.V FLOPs)", "ms_per_step": round(step_ms, 4), "steps": steps,
           "mainloop_ms": round(main_ms, 4), "prep_ms": round(prep_ms, 4),
           "mainloop_TOPS": round(loop_tops, 2),
           "frac_of_int8_fp8_peak": round(tops / Q8_PEAK_TOPS, 4),
           "path": "quant (int8 QK, fp8 PV)", "step_ms_dist": dist,
           "roofline": {"bound": "mfma", "achieved": round(loop_tops, 2), "peak": Q8_PEAK_TOPS, "unit": "TOPS",
                        "frac": round(loop_tops / Q8_PEAK_TOPS, 4),
                        "traffic": measured_traffic(QUANT_SOURCES, "quant_attn_kernel__dit_quant.traffic.json"),
                        "kernel": "quant_attn_kernel", "kernel_ms": round(main_ms, 4)}}
    if cpu_seconds > 0:
        log("[bench] timing the quantised CPU oracle on a sample")
        res["cpu_baseline"] = cpu_quant_baseline(case, cpu_seconds)
        log("[bench] cpu baseline %s" % json.dumps(res["cpu_baseline"]))
    return res


# the sources each kernel is built from: a counter summary taken on other
# sources no longer describes the kernel
DECODE_SOURCES = ["decode_kernels.h", "decode_split.hip", "attn_device.h", "kv_quant.h"]
PREFILL_SOURCES = ["prefill.hip", "attn_device.h", "kv_quant.h", "lds_stream.h"]
QUANT_SOURCES = ["quant.hip", "attn_device.h", "quant_device.h", "lds_stream.h"]


def measured_traffic(kernel_files, profile_name):
    """HBM bytes per launch of the dominant kernel from the committed
    FETCH_SIZE / WRITE_SIZE counter summary, each scaled by what the same
    counter read for a plain 1 GiB copy.  None when no summary exists or the
    kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    h = hashlib.sha1()
    for f in kernel_files:
        h.update(open(os.path.join(ROOT, "paged_kv_gqa_fwd_amd", "csrc", f), "rb").read())
    if h.hexdigest() != d.get("kernel_sources_sha1"):
        return None
    copy_kib = d["copy_bytes_per_dispatch"] / 1024.0
    fetch = d["fetch_kib_per_dispatch"] * copy_kib / d["copy_fetch_kib_per_dispatch"]
    write = d["write_kib_per_dispatch"] * copy_kib / d["copy_write_kib_per_dispatch"]
    return round((fetch + write) * 1024.0)


def _roofline(res, bound):
    """Roofline block of a line's dominant kernel: algorithmic bytes (or
    FLOPs) per launch over its average launch duration from the library's
    HIP events on the launch stream."""
    name = res["workload"]
    kern = ("paged_decode_balanced_kernel" if res["path"].startswith("balanced") else
            "paged_decode_split_kernel" if "split" in res["path"] else "paged_prefill_kernel")
    if bound == "hbm":
        ach = res["bytes"] / (res["main_kernel_ms"] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kern,
                "kernel_ms": round(res["main_kernel_ms"], 4)}
    ach = res["flops"] / (res["main_kernel_ms"] * 1e-3) / 1e12
    traffic = None
    if name == "chunked_prefill" or name == "dit_self_attn":
        traffic = measured_traffic(PREFILL_SOURCES,
                                   "paged_prefill_kernel__%s.traffic.json" % name)
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": kern,
            "kernel_ms": round(res["main_kernel_ms"], 4)}


def summarize(res):
    name = res["workload"]
    base = name.split("+")[0]
    if base == "tiny_mixed":
        # the manifest's tiny mixed call: its working set (about 3 MB) sits in
        # the caches, so the line reports latency
        us = res["ms_per_step"] * 1e3
        return {"workload": name, "value": round(us, 2), "unit": "us per call (latency)",
                "ms_per_step": round(res["ms_per_step"], 4), "steps": res["steps"],
                "main_kernel_ms": round(res["main_kernel_ms"], 4), "path": res["path"],
                "step_ms_dist": res.get("step_ms_dist"),
                "algorithmic_flops": res["flops"], "algorithmic_bytes": res["bytes"],
                "roofline": _roofline(res, "hbm")}
    if BOUND[base] == "hbm":
        val = res["bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
        kern = res["bytes"] / (res["main_kernel_ms"] * 1e-3) / 1e9
        return {"workload": name, "value": round(val, 2), "unit": "GB/s",
                "frac_of_peak": round(val / HBM_PEAK_GBS, 4), "ms_per_step": round(res["ms_per_step"], 4),
                "steps": res["steps"], "main_kernel_ms": round(res["main_kernel_ms"], 4),
                "combine_kernel_ms": round(res["combine_kernel_ms"], 4),
                "main_kernel_GBps": round(kern, 2), "path": res["path"],
                "pages_per_split": res["pages_per_split"], "max_splits": res["max_splits"],
                "step_ms_dist": res.get("step_ms_dist"), "roofline": _roofline(res, "hbm")}
    val = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12
    return {"workload": name, "value": round(val, 2), "unit": "TFLOP/s",
            "frac_of_peak": round(val / BF16_PEAK_TFLOPS, 4), "ms_per_step": round(res["ms_per_step"], 4),
            "steps": res["steps"], "main_kernel_ms": round(res["main_kernel_ms"], 4), "path": res["path"],
            "step_ms_dist": res.get("step_ms_dist"), "roofline": _roofline(res, "mfma")}


# ---------------------------------------------------------------- CPU oracle
def _grow_and_time(run, max_seconds, start=1, limit=None):
    """Time run(k) on growing samples k (doubling from `start`, at most
    `limit`) until one pass takes a quarter of max_seconds or the sample is
    the whole workload, then repeat passes to about max_seconds in total.
    Returns (k, seconds per pass, passes)."""
    k = start
    while True:
        t = time.perf_counter()
        run(k)
        t_one = time.perf_counter() - t
        if t_one > max_seconds / 4 or (limit is not None and k >= limit):
            break
        k = k * 2 if limit is None else min(limit, k * 2)
    reps = max(1, min(50, int(max_seconds / max(t_one, 1e-3))))
    t = time.perf_counter()
    for _ in range(reps):
        run(k)
    return k, (time.perf_counter() - t) / reps, reps


def _oracle_info():
    import oracle
    return {"cores": oracle.num_threads(), "kind": "oracle", "cpu": _cpu_model(), "nproc": os.cpu_count()}


def cpu_decode_baseline(case, name, max_seconds):
    """ORACLE-P on a prefix of the batch's sequences, in GB/s of the
    prefix's algorithmic bytes."""
    import oracle
    state = {}

    def run(k):
        state["sub"] = sub = _prefix_case(case, k)
        oracle.paged_attn(sub.q, sub.kv, sub.block_table, sub.seq_lens, sub.cu_q, sub.scale, sub.causal)

    k, t_used, reps = _grow_and_time(run, max_seconds, 1, case.n_seqs)
    sub = state["sub"]
    info = _oracle_info()
    return dict(value=round(algorithmic_bytes(sub) / t_used / 1e9, 4), unit="GB/s",
                sample="first %d of %d sequences of the %s workload, %d timed passes of %.3f s each "
                       "(fp64 oracle, OpenMP threads=%d)" % (k, case.n_seqs, name, reps, t_used, info["cores"]),
                **info)


def cpu_prefill_baseline(case, name, max_seconds, seed=11):
    """ORACLE-P on a seeded sample of token rows (every head of each), in
    TFLOP/s of the sample's algorithmic FLOPs (4 D per visible (query, q
    head, key))."""
    import numpy as np
    import oracle
    c = case.to("cpu")
    T = sum(c.q_lens)
    order = torch.randperm(T, generator=torch.Generator().manual_seed(seed)).numpy()
    state = {}

    def run(k):
        mask = np.zeros(T, dtype=np.uint8)
        mask[order[:k]] = 1
        state["mask"] = mask
        oracle.paged_attn(c.q, c.kv, c.block_table, c.seq_lens, c.cu_q, c.scale, c.causal, row_mask=mask)

    k, t_used, reps = _grow_and_time(run, max_seconds, 4, T)
    rows = np.nonzero(state["mask"])[0]
    vis = 0
    cu = c.cu_q.tolist()
    for t in rows.tolist():
        b = next(i for i in range(c.n_seqs) if cu[i] <= t < cu[i + 1])
        n, L, i = c.q_lens[b], c.kv_lens[b], t - cu[b]
        vis += max(0, min(L, L - n + i + 1)) if c.causal else L
    flops = 4 * c.head_dim * c.num_q_heads * vis
    info = _oracle_info()
    del c
    return dict(value=round(flops / t_used / 1e12, 6), unit="TFLOP/s",
                sample="%d seeded token rows (all %d heads) of %d in the %s workload, %d timed passes of %.3f s "
                       "each (fp64 oracle, OpenMP threads=%d)" % (k, case.num_q_heads, T, name, reps, t_used,
                                                                  info["cores"]), **info)


def cpu_quant_baseline(case, max_seconds, seed=11):
    """ORACLE-Q: its preparation over the whole DiT shape (one pass) plus its
    attention on a seeded sample of query tokens; the whole path's time is
    estimated as prep + sample time x (N / sample), reported in T ops/s of
    the path's algorithmic work."""
    import numpy as np
    import oracle
    q, k, v = (t.cpu() for t in workloads.dense_from_case(case))
    t = time.perf_counter()
    prep = oracle.quant_prep(q, k, v)
    prep_s = time.perf_counter() - t
    N = q.shape[1]
    order = torch.randperm(N, generator=torch.Generator().manual_seed(seed)).numpy()

    def run(kk):
        mask = np.zeros(N, dtype=np.uint8)
        mask[order[:kk]] = 1
        oracle.quant_attn(prep, case.scale, False, row_mask=mask)

    kk, t_used, reps = _grow_and_time(run, max(1.0, max_seconds - prep_s), 2, N)
    full_s = prep_s + t_used * N / kk
    flops = algorithmic_flops(case)
    info = _oracle_info()
    return dict(value=round(flops / full_s / 1e12, 6), unit="TOPS (int8 Q.K ops + fp8 P.V FLOPs)",
                prep_s=round(prep_s, 3), attention_s_per_token=round(t_used / kk, 6),
                sample="preparation over all %d tokens (%.2f s) + attention on %d seeded query tokens (all %d "
                       "heads), %d timed passes of %.3f s; the whole path's time estimated as prep + that x %d/%d "
                       "(fp64 quantisation-emulating oracle, OpenMP threads=%d)"
                       % (N, prep_s, kk, case.num_q_heads, reps, t_used, N, kk, info["cores"]), **info)


def cpu_baseline(res, max_seconds=20.0):
    """The fp64 CPU oracle on a bounded sample of a line's workload, in the
    line's unit (decode: a prefix of the batch; prefill: sampled rows)."""
    case, name = res["case"], res["workload"]
    base = name.split("+")[0]
    if BOUND[base] == "hbm" and base != "tiny_mixed":
        return cpu_decode_baseline(case, name, max_seconds)
    if base == "tiny_mixed":
        import oracle
        c = case.to("cpu")

        def run(_k):
            oracle.paged_attn(c.q, c.kv, c.block_table, c.seq_lens, c.cu_q, c.scale, c.causal)

        _, t_used, reps = _grow_and_time(run, max_seconds, 1, 1)
        info = _oracle_info()
        return dict(value=round(t_used * 1e6, 1), unit="us per call (latency)",
                    sample="the whole tiny mixed call, %d timed passes (fp64 oracle, OpenMP threads=%d)"
                           % (reps, info["cores"]), **info)
    return cpu_prefill_baseline(case, name, max_seconds)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _prefix_case(case, k):
    """CPU copy of the first k sequences (pages gathered into a compact pool)."""
    from dataclasses import replace
    bt = case.block_table.cpu()
    P = case.kv.shape[1]
    pages, rows = [], []
    for b in range(k):
        npg = (case.kv_lens[b] + P - 1) // P
        ids = bt[b, :npg].tolist()
        rows.append(list(range(len(pages), len(pages) + npg)) + [-1] * (bt.shape[1] - npg))
        pages.extend(ids)
    kv = case.kv.index_select(0, torch.tensor(pages, dtype=torch.long, device=case.kv.device)).cpu()
    T = sum(case.q_lens[:k])
    return replace(case, q=case.q[:T].cpu(), kv=kv, pool_storage=kv,
                   block_table=torch.tensor(rows, dtype=torch.int32),
                   seq_lens=case.seq_lens[:k].cpu(), cu_q=case.cu_q[:k + 1].cpu(),
                   q_lens=case.q_lens[:k], kv_lens=case.kv_lens[:k])


def calibrate_gemm(n=16384, iters=20):
    """Vendor GEMM throughput (hipBLASLt through torch) at n x n x n.  MFMA
    power depends on the data: random operands run at a lower clock than
    constant ones, so the random-data rate is the practical ceiling."""
    g = torch.Generator(device="cuda").manual_seed(0)

    def rate(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(2.0 * n ** 3 / (e0.elapsed_time(e1) / iters) / 1e9, 1)

    res = {"calibration": "gemm", "n": n, "unit": "T(FL)OP/s"}
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    res["bf16_random"] = rate(lambda: a @ b)
    c = torch.ones_like(a)
    res["bf16_constant"] = rate(lambda: c @ c)
    del c
    try:
        ai = torch.randint(-127, 128, (n, n), device="cuda", dtype=torch.int8, generator=g)
        bi = torch.randint(-127, 128, (n, n), device="cuda", dtype=torch.int8, generator=g)
        res["int8_random"] = rate(lambda: torch._int_mm(ai, bi))
        del ai, bi
    except Exception as e:  # the library may not cover this type on the platform
        res["int8_random"] = "unavailable: %s" % type(e).__name__
    try:
        af = a.to(torch.float8_e4m3fn)
        bf = b.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device="cuda")
        res["fp8_random"] = rate(lambda: torch._scaled_mm(af, bf, one, one, out_dtype=torch.bfloat16))
    except Exception as e:
        res["fp8_random"] = "unavailable: %s" % type(e).__name__
    print(json.dumps(res), flush=True)


SECONDARY = ("tiny_mixed,long_decode,long_decode+slot_major,chunked_prefill,chunked_prefill+fp8,dit_self_attn,"
             "dit_quant,short_batch,short_batch+prefill,chunked_prefill+kv_write,long_decode+window4096,"
             "long_decode+fp8,decode_batch+fp8,decode_batch+kv_write")
# secondary lines that carry the CPU oracle (the configurations themselves;
# their window / fp8 / layout / write variants do not)
CPU_LINES = {"tiny_mixed": 3.0, "long_decode": 6.0, "chunked_prefill": 6.0, "dit_self_attn": 6.0, "dit_quant": 8.0}


def run_secondary(name, args, cpu_on):
    """One secondary line (time-bounded warmup of at least W calls, about
    0.4 s of timed calls), with its CPU oracle where CPU_LINES names it."""
    W, K = args.warmup, args.steps
    cpu_s = CPU_LINES.get(name, 0.0) if cpu_on else 0.0
    if name.endswith("+kv_write"):
        return run_write(name[:-len("+kv_write")], K, W)
    if name == "dit_quant":
        return run_quant(K, W, cpu_seconds=cpu_s)
    kw = {}
    base = name
    if name.endswith("+fp8"):
        base, kw["fp8"] = name[:-len("+fp8")], True
    elif "+window" in name:
        base, w = name.split("+window")
        kw["window"] = int(w)
    elif name.endswith("+slot_major") or name.endswith("+head_major"):
        base, kw["layout"] = name.split("+")
    if name.endswith("+prefill"):
        # the same workload forced onto the prefill kernel: the route that
        # short query runs took before the short-sequence body
        base, path = name[:-len("+prefill")], 2
        kw["tag"] = "+prefill"
    else:
        path = args.path if args.path != 2 and BOUND[base] == "hbm" and base != "tiny_mixed" else 0   # 2 = prefill
    r = run_workload(base, K, W, path=path, **kw)
    ss = summarize(r)
    if cpu_s > 0:
        log("[bench] timing the CPU oracle on a sample of %s" % name)
        ss["cpu_baseline"] = cpu_baseline(r, cpu_s)
    del r
    return ss


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_batch", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--secondary", default=SECONDARY, help="comma list of extra workloads to time ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--path", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (torch copy_) five times: "
                         "the reference for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--calibrate-gemm", action="store_true",
                    help="run only the vendor library's large GEMMs (bf16 on random and on constant "
                         "data, int8, fp8) and print their throughput: the MFMA rate the chip "
                         "sustains on real data, as context for the prefill and quantised rooflines")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n,
                          "bytes_written_per_launch": n, "launches": 5}), flush=True)
        return
    if args.calibrate_gemm:
        calibrate_gemm()
        return
    torch.manual_seed(0)
    cpu_on = not args.no_cpu_baseline
    # The primary line first (W warmup and K timed steps right after its
    # inputs are generated, before the secondary lines have heated the chip:
    # the decode kernel, mostly HBM-bound, measured 1-3% slower at the end of
    # the run than at its start), then the secondary lines.
    prim = run_workload(args.workload, args.steps, args.warmup, args.pages_per_split, args.path, secondary=False)
    s = summarize(prim)
    log("[bench] %s" % json.dumps(s))
    bound = BOUND[args.workload]
    roof = s["roofline"]
    if bound == "hbm" and args.workload == "decode_batch" and "split" in prim["path"]:
        roof["traffic"] = measured_traffic(DECODE_SOURCES,
                                           "%s__decode_batch.traffic.json" % roof["kernel"])
    ceiling = None
    if bound == "hbm":
        # the practical denominator beside the 8 TB/s peak: a plain read
        # stream over as many bytes as one step moves, right after the
        # primary line (the same state of the chip)
        ceiling = stream_read_ceiling(prim["bytes"])
        if "main_kernel_GBps" in s:   # split-decode lines (the tiny call runs the prefill kernel)
            ceiling["kernel_frac"] = round(s["main_kernel_GBps"] / ceiling["GBps"], 4)
        ceiling["step_frac"] = round(s["value"] / ceiling["GBps"], 4)
        log("[bench] read ceiling %s" % json.dumps(ceiling))
    cpu = None
    if cpu_on:
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(prim)
        log("[bench] cpu baseline %s" % json.dumps(cpu))
    case = prim["case"]
    secondary = []
    for name in [x for x in args.secondary.split(",") if x and x != args.workload]:
        ss = run_secondary(name, args, cpu_on)
        log("[bench] %s" % json.dumps(ss))
        secondary.append(ss)
        torch.cuda.empty_cache()
    line = {
        "metric": METRIC, "value": s["value"], "unit": s["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(prim["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled page pool)",
        "config": {"workload": DESCR[args.workload], "n_seqs": case.n_seqs,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "page_size": 64, "total_kv_tokens": sum(case.kv_lens),
                   "algorithmic_bytes": prim["bytes"], "algorithmic_flops": prim["flops"], "path": prim["path"],
                   "pages_per_split": prim["pages_per_split"], "max_splits": prim["max_splits"]},
        "frac_of_peak": s.get("frac_of_peak"),
        "roofline": roof,
        "read_ceiling": ceiling,
        "step_ms_dist": s.get("step_ms_dist"),
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
