"""Benchmark of the paged GQA attention hot path on one MI355X.

One "step" is one full forward pass (all kernels of the path: split-KV decode
partials + log-sum-exp combine, or the prefill kernel) over one batch of
synthetic, seeded input already resident in HBM.

Default workload: the decode batch (64 sequences x 1 query token, 32 q / 8 KV
heads, head_dim 128, page 64, KV lengths uniform in [1024, 8192], causal),
reported as achieved HBM GB/s of algorithmic bytes (K and V read once per KV
head, plus Q and the output).  Secondary lines (long-context decode, chunked
prefill, DiT non-causal) are reported alongside, prefill ones in TFLOP/s of
algorithmic FLOPs (4 * D per visible (query, q head, key) triple).

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
}
BOUND = {"decode_batch": "hbm", "long_decode": "hbm", "chunked_prefill": "mfma",
         "dit_self_attn": "mfma", "tiny_mixed": "hbm"}


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
    mm, mn, cm, cn, pm, pn = pa.kernel_timing_read()
    return mm / max(mn, 1), (cm / cn if cn else 0.0), (pm / pn if pn else 0.0)


# Nominal ms per step of each workload on MI355X: bounds the secondary lines'
# step counts so that each times about a third of a second.
NOMINAL_MS = {"decode_batch": 0.25, "long_decode": 1.5, "chunked_prefill": 4.0, "dit_self_attn": 40.0,
              "dit_quant": 25.0, "tiny_mixed": 0.05}


def sec_counts(name, steps, warmup):
    per = NOMINAL_MS.get(name.split("+")[0], 1.0)
    return max(3, min(steps // 2, int(300.0 / per))), max(1, min(warmup // 2, int(100.0 / per)))


def run_workload(name, steps, warmup, pps=0, path=0, window=0, fp8=False):
    import paged_kv_gqa_fwd_amd as pa
    log("[bench] generating %s%s%s" % (name, " (window %d)" % window if window else "", " (fp8 cache)" if fp8 else ""))
    case = workloads.WORKLOADS[name](device="cuda")
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

    for _ in range(warmup):
        step()
    step_ms = _time_steps(step, steps)
    main_ms, comb_ms, _ = _kernel_times(step, steps)
    dist = _step_distribution(step, steps)
    res = {
        "workload": name + ("+window%d" % window if window else "") + ("+fp8" if fp8 else ""), "case": case,
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
    for every query token.  The line's value is the write kernel's rate:
    every new K/V byte read once and written once."""
    import paged_kv_gqa_fwd_amd as pa
    log("[bench] generating %s (with KV-cache write)" % name)
    case = workloads.WORKLOADS[name](device="cuda")
    k_new, v_new = workloads.new_kv_tokens(case, case.seed + 1000)
    out = torch.empty_like(case.q)

    def step():
        pa.paged_attention_write(case.q, k_new, v_new, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                 max(case.max_q, 1), case.scale, case.causal, out=out)

    for _ in range(warmup):
        step()
    step_ms = _time_steps(step, steps)
    main_ms, comb_ms, write_ms = _kernel_times(step, steps)
    written = sum(min(n, L) for n, L in zip(case.q_lens, case.kv_lens))
    wbytes = 2 * written * case.num_kv_heads * 2 * case.head_dim * 2
    return {"workload": name + "+kv_write", "value": round(wbytes / (write_ms * 1e-3) / 1e9, 2),
            "unit": "GB/s (write kernel)", "write_bytes": wbytes, "write_kernel_ms": round(write_ms, 4),
            "ms_per_step": round(step_ms, 4), "attention_ms": round(main_ms + comb_ms, 4),
            "path": "kv_write + attention"}


def run_quant(steps, warmup):
    """The quantised path (attn_quant_fwd: preparation + fused int8/fp8 loop)
    on the video-DiT shape, same seeded Q/K/V as the bf16 DiT workload."""
    import paged_kv_gqa_fwd_amd as pa
    log("[bench] generating dit_self_attn (quantised path)")
    case = workloads.dit_self_attn(device="cuda")
    q, k, v = workloads.dense_from_case(case)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

    def step():
        pa.quant_attention(q, k, v, case.scale, False, out=out)

    for _ in range(warmup):
        step()
    step_ms = _time_steps(step, steps)
    main_ms, _, prep_ms = _kernel_times(step, steps)
    flops = algorithmic_flops(case)
    return {"workload": "dit_quant", "value": round(flops / (step_ms * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s", "ms_per_step": round(step_ms, 4),
            "mainloop_ms": round(main_ms, 4), "prep_ms": round(prep_ms, 4),
            "mainloop_TOPS": round(flops / (main_ms * 1e-3) / 1e12, 2),
            "frac_of_int8_fp8_peak": round(flops / (step_ms * 1e-3) / 1e12 / Q8_PEAK_TOPS, 4),
            "path": "quant (int8 QK, fp8 PV)"}


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


def summarize(res):
    name = res["workload"]
    if BOUND[name.split("+")[0]] == "hbm":
        val = res["bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
        kern = res["bytes"] / (res["main_kernel_ms"] * 1e-3) / 1e9
        return {"workload": name, "value": round(val, 2), "unit": "GB/s",
                "frac_of_peak": round(val / HBM_PEAK_GBS, 4), "ms_per_step": round(res["ms_per_step"], 4),
                "main_kernel_ms": round(res["main_kernel_ms"], 4),
                "combine_kernel_ms": round(res["combine_kernel_ms"], 4),
                "main_kernel_GBps": round(kern, 2), "path": res["path"],
                "pages_per_split": res["pages_per_split"], "max_splits": res["max_splits"],
                "step_ms_dist": res.get("step_ms_dist")}
    val = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12
    return {"workload": name, "value": round(val, 2), "unit": "TFLOP/s",
            "frac_of_peak": round(val / BF16_PEAK_TFLOPS, 4), "ms_per_step": round(res["ms_per_step"], 4),
            "main_kernel_ms": round(res["main_kernel_ms"], 4), "path": res["path"],
            "step_ms_dist": res.get("step_ms_dist")}


def cpu_baseline(res, max_seconds=20.0):
    """Time the fp64 CPU oracle on a bounded sample of the primary workload
    (a prefix of its sequences) and report the same metric's unit."""
    import oracle
    from dataclasses import replace
    case = res["case"]
    name = res["workload"]
    nthreads = oracle.num_threads()
    # grow the sample (a prefix of the batch) until one pass takes a few
    # seconds or covers the batch, then repeat passes to ~max_seconds in total
    k = 1
    while True:
        sub = _prefix_case(case, k)
        t = time.perf_counter()
        oracle.paged_attn(sub.q, sub.kv, sub.block_table, sub.seq_lens, sub.cu_q, sub.scale,
                          sub.causal)
        t_one = time.perf_counter() - t
        if t_one > max_seconds / 4 or k >= case.n_seqs:
            break
        k = min(case.n_seqs, k * 2)
    reps = max(1, min(50, int(max_seconds / max(t_one, 1e-3))))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.paged_attn(sub.q, sub.kv, sub.block_table, sub.seq_lens, sub.cu_q, sub.scale,
                          sub.causal)
    t_used = (time.perf_counter() - t) / reps
    if BOUND[name] == "hbm":
        val = algorithmic_bytes(sub) / t_used / 1e9
        unit = "GB/s"
    else:
        val = algorithmic_flops(sub) / t_used / 1e12
        unit = "TFLOP/s"
    return {"value": round(val, 4), "unit": unit, "cores": nthreads, "kind": "oracle",
            "sample": "first %d of %d sequences of the %s workload, %d timed passes of %.3f s each "
                      "(fp64 oracle, OpenMP threads=%d)" % (k, case.n_seqs, name, reps, t_used, nthreads),
            "cpu": _cpu_model(), "nproc": os.cpu_count()}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_batch", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--secondary", default="long_decode,chunked_prefill,dit_self_attn,dit_quant,"
                                           "decode_batch+kv_write,chunked_prefill+kv_write,long_decode+window4096,"
                                           "decode_batch+fp8,long_decode+fp8",
                    help="comma list of extra workloads to time ('' for none)")
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
    prim = run_workload(args.workload, args.steps, args.warmup, args.pages_per_split, args.path)
    s = summarize(prim)
    log("[bench] %s" % json.dumps(s))
    secondary = []
    for name in [x for x in args.secondary.split(",") if x and x != args.workload]:
        if name.endswith("+fp8"):
            r = run_workload(name[:-len("+fp8")], *sec_counts(name, args.steps, args.warmup), fp8=True)
            ss = summarize(r)
            log("[bench] %s" % json.dumps(ss))
            secondary.append(ss)
            del r
            torch.cuda.empty_cache()
            continue
        if "+window" in name:
            base, w = name.split("+window")
            r = run_workload(base, *sec_counts(name, args.steps, args.warmup), window=int(w))
            ss = summarize(r)
            log("[bench] %s" % json.dumps(ss))
            secondary.append(ss)
            del r
            torch.cuda.empty_cache()
            continue
        if name.endswith("+kv_write"):
            ss = run_write(name[:-len("+kv_write")], *sec_counts(name, args.steps, args.warmup))
            log("[bench] %s" % json.dumps(ss))
            secondary.append(ss)
            torch.cuda.empty_cache()
            continue
        if name == "dit_quant":
            ss = run_quant(*sec_counts(name, args.steps, args.warmup))
            log("[bench] %s" % json.dumps(ss))
            secondary.append(ss)
            torch.cuda.empty_cache()
            continue
        sec_path = args.path if args.path != 2 and BOUND[name] == "hbm" else 0   # 2 = prefill
        r = run_workload(name, *sec_counts(name, args.steps, args.warmup), path=sec_path)
        ss = summarize(r)
        log("[bench] %s" % json.dumps(ss))
        secondary.append(ss)
        del r
        torch.cuda.empty_cache()
    bound = BOUND[args.workload]
    if bound == "hbm":
        traffic = None
        kname = ("paged_decode_balanced_kernel" if prim["path"].startswith("balanced") else
                 "paged_decode_split_kernel" if "split" in prim["path"] else "paged_prefill_kernel")
        if args.workload == "decode_batch" and "split" in prim["path"]:
            traffic = measured_traffic(["decode_split.hip", "attn_device.h"],
                                       "%s__decode_batch.traffic.json" % kname)
        roof = {"bound": "hbm", "achieved": s["main_kernel_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(s["main_kernel_GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kname, "kernel_ms": s["main_kernel_ms"]}
    else:
        ach = prim["flops"] / (prim["main_kernel_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "paged_prefill_kernel", "kernel_ms": s["main_kernel_ms"]}
    ceiling = None
    if bound == "hbm":
        # the practical denominator beside the 8 TB/s peak: a plain read
        # stream over as many bytes as one step moves
        ceiling = stream_read_ceiling(prim["bytes"])
        ceiling["kernel_frac"] = round(s["main_kernel_GBps"] / ceiling["GBps"], 4)
        ceiling["step_frac"] = round(s["value"] / ceiling["GBps"], 4)
        log("[bench] read ceiling %s" % json.dumps(ceiling))
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(prim)
        log("[bench] cpu baseline %s" % json.dumps(cpu))
    case = prim["case"]
    line = {
        "metric": METRIC, "value": s["value"], "unit": s["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(prim["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled page pool)",
        "config": {"workload": DESCR[args.workload], "n_seqs": case.n_seqs,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "page_size": 64, "total_kv_tokens": sum(case.kv_lens),
                   "algorithmic_bytes": prim["bytes"], "path": prim["path"],
                   "pages_per_split": prim["pages_per_split"], "max_splits": prim["max_splits"]},
        "frac_of_peak": s["frac_of_peak"],
        "roofline": roof,
        "read_ceiling": ceiling,
        "step_ms_dist": s.get("step_ms_dist"),
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
