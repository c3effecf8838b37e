#!/usr/bin/env python3
"""Benchmark of MLA chunked-context prefill on one MI355X.

One step = the whole hot path over one batch: host planning and the metadata
upload, then per chunk gather -> chunk attention -> accumulate, the causal
suffix attention and the final merge (mla_chunked_prefill).  Inputs are
synthetic and already resident in HBM when the timed region starts.

Prints one JSON line.  `value` is the whole step's attention throughput:
algorithmic flops of chunk + suffix attention per second (2*(192+128) flops
per unmasked (query, key, head)).  `roofline` is for the dominant kernel
(the kernel kind with the most time), timed live with HIP events on its own
stream over the timed region.  `cpu_baseline` times the fp64 oracle on a
bounded sample of the same workload on the host cores.

--path uniform_window times the earlier equal-window scheduler
(mla_uniform_window_prefill) instead and also times the chunked path on the
same batch, reporting both latencies.  --path mask_empty_context times the
empty-context mask alone (one launch over the batch per step).  --path dcp
times mla_dcp_chunked_prefill with the context sharded over --dcp-world
emulated ranks (every rank's local gather runs on this one GPU), beside the
single-device path on the same batch.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunk-attn TFLOP/s + merge GB/s (% roofline); chunked-prefill latency ms"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
FLOP_PER_PAIR = 2 * (192 + 128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_figures(wl, chunks, windows=None):
    H = wl.num_heads
    ctx = wl.context_lens
    ql = wl.query_lens
    chunk_flops = FLOP_PER_PAIR * H * sum(q * c for q, c in zip(ql, ctx))
    suffix_flops = FLOP_PER_PAIR * H * sum(q * (q + 1) // 2 for q in ql)
    rows = sum(ctx)
    gather_bytes = 2 * H * (192 + 128) * 2 * rows  # read + write of bf16 K and V rows
    T = wl.num_tokens
    merge_row = 3 * (128 * 2 + 4)  # read two (row, LSE) states, write one
    final_merge_bytes = T * H * merge_row
    cont_rows = sum(ql[c["request_begin"]] for c in chunks if c["is_continuation"])
    accumulate_bytes = cont_rows * H * merge_row
    mask_bytes = 0
    if windows is not None:  # uniform-window scheduler: whole-batch merges and masks
        accumulate_bytes = max(0, len(windows) - 1) * T * H * merge_row
        qsl = [0]
        for x in ql:
            qsl.append(qsl[-1] + x)
        for lens in windows:
            if any(x == 0 for x in lens):
                rows = sum(ql[r] for r in range(len(ql)) if lens[r] == 0)
                mask_bytes += rows * H * (128 * 2 + 4) + (len(ql) + 1) * 8
    # chunk attention must read Q, the gathered K/V rows and write O + LSE
    if windows is None:
        q_rows = sum(sum(ql[c["request_begin"]:c["request_end"]]) for c in chunks)
    else:
        q_rows = len(windows) * T
    chunk_bytes = H * (q_rows * (192 * 2 + 128 * 2 + 4) + rows * (192 + 128) * 2)
    return dict(chunk_flops=chunk_flops, suffix_flops=suffix_flops, gather_bytes=gather_bytes, chunk_bytes=chunk_bytes,
                merge_bytes=final_merge_bytes + accumulate_bytes, final_merge_bytes=final_merge_bytes,
                accumulate_bytes=accumulate_bytes, mask_bytes=mask_bytes)


def profiled_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter profile, if
    it was taken on this workload and the kernel's sources are unchanged since
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    k = prof.get("kernels", {}).get(kernel)
    if k is None:
        return None
    h = hashlib.sha256()
    for src in k["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != k["source_sha256"]:
        return None
    return k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"]


# sources whose hash a kernel's traffic figure is tied to (besides device.h)
ATTN_SOURCES = ["attention.hip", "work_queues.h"]
TRAFFIC_SOURCES = {"chunk_attention_kernel": ATTN_SOURCES, "suffix_attention_kernel": ATTN_SOURCES,
                   "chunk_attention_queued_kernel": ATTN_SOURCES, "suffix_attention_queued_kernel": ATTN_SOURCES}


def write_traffic(fetch_csv, write_csv, workload, out_path=None):
    """profiles/<workload>_traffic.json from two rocprofv3 counter collections
    (--pmc FETCH_SIZE and --pmc WRITE_SIZE of a run with
    --calibration-copy-mb 1024).  Each counter is scaled by the bytes per
    counter unit of the run's 1 GiB elementwise copy (the torch negation
    launched after the timed steps); the library's kernels get their mean
    bytes per launch and a hash of their sources.  Host only."""
    import collections
    import csv
    import hashlib

    def per_kernel(path, counter):
        disp = collections.defaultdict(float)
        names = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = int(r["Dispatch_Id"])
                names[k] = r["Kernel_Name"]
                disp[k] += float(r["Counter_Value"])
        out = collections.defaultdict(list)
        for k, v in disp.items():
            n = names[k]
            if n.startswith("void "):  # function templates demangle with their return type
                n = n[len("void "):]
            if "neg_kernel" in n:
                out["calibration"].append(v)
            elif n.startswith("mla::"):
                short = n.replace("(anonymous namespace)::", "").split("(")[0].split("::")[-1].split("<")[0]
                out[short].append(v)
        return out

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    if len(fetch["calibration"]) != 1 or len(write["calibration"]) != 1:
        raise SystemExit("expected exactly one calibration copy dispatch in each counter collection")
    gib = float(1 << 30)
    fetch_scale = gib / (fetch["calibration"][0] * 1024)
    write_scale = gib / (write["calibration"][0] * 1024)
    res = {"workload": workload,
           "how": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch), each scaled by the "
                  "counter-per-byte ratio of a 1 GiB elementwise copy run in the same process",
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4), "kernels": {}}
    for k in sorted(set(fetch) - {"calibration"}):
        if not write.get(k):
            continue
        srcs = [f"mla_chunked_context_amd/csrc/{f}" for f in TRAFFIC_SOURCES.get(k, ["memory_ops.hip"])] + \
            ["mla_chunked_context_amd/csrc/device.h"]
        h = hashlib.sha256()
        for src in srcs:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        res["kernels"][k] = {
            "launches_profiled": len(fetch[k]),
            "fetch_bytes_per_launch": int(sum(fetch[k]) / len(fetch[k]) * 1024 * fetch_scale),
            "write_bytes_per_launch": int(sum(write[k]) / len(write[k]) * 1024 * write_scale),
            "source_sha256": h.hexdigest(), "sources": srcs}
    path = out_path or os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    log(f"bench: wrote {path}")
    return res


def host_cpus():
    """(worker threads, machine CPUs, CPU model) of this host.  Workers: the
    CPUs this process may run on, capped by OMP_NUM_THREADS when it is set
    (a GPU machine gives each GPU a share of the host's cores)."""
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS")
    workers = min(usable, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else usable
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return workers, os.cpu_count() or usable, model


# default oracle sample per workload: (heads, query tokens per request); None = all
ORACLE_SAMPLE = {"long_context": ("workers", 2048), "heterogeneous": ("workers", None), "skewed": ("workers", 128)}


def cpu_baseline(b, wl, path="chunked", rank_caches=None, dcp=(1, 1), sample_heads=None, sample_queries=None):
    """The oracle's whole path (fp64 NumPy: plan, gather, context attention,
    merges, causal suffix, final merge) timed on the host cores.  Work items
    are heads (the path is independent per head): a pool of one thread per
    core runs one head's path per item with one BLAS thread each.  Inputs are
    host copies made before timing (resident, as on the GPU).  Workloads too
    large to run whole are sampled (a seeded subset of heads and/or the first
    tokens of every request); the full step's time is then scaled by flops
    and labelled "extrapolated"."""
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W

    workers, machine_cpus, model = host_cpus()
    H = wl.num_heads
    d_heads, d_queries = ORACLE_SAMPLE.get(wl.name, (None, None))
    if sample_heads is None:
        sample_heads = min(H, workers) if d_heads == "workers" else H
    if sample_queries is None:
        sample_queries = d_queries
    heads = sorted(int(h) for h in np.random.default_rng(0).choice(H, size=min(H, sample_heads), replace=False))
    sq = [q if sample_queries is None else min(sample_queries, q) for q in wl.query_lens]
    qsl = np.concatenate([[0], np.cumsum(wl.query_lens)])
    idx = np.concatenate([np.arange(qsl[r], qsl[r] + sq[r]) for r in range(wl.num_requests)] + [np.zeros(0)])
    it = torch.from_numpy(idx.astype(np.int64)).to(b.q.device)
    f = W.to_f64
    table = b.block_table.cpu().numpy()

    def inputs(h):
        hs = slice(h, h + 1)
        q = f(b.q.index_select(0, it)[:, hs].contiguous())
        kn = f(b.k_new.index_select(0, it)[:, hs].contiguous())
        vn = f(b.v_new.index_select(0, it)[:, hs].contiguous())
        if path == "dcp":
            return (q, kn, vn, [f(r.k_cache[:, :, hs].contiguous()) for r in rank_caches],
                    [f(r.v_cache[:, :, hs].contiguous()) for r in rank_caches],
                    [r.block_table.cpu().numpy() for r in rank_caches])
        return q, kn, vn, f(b.k_cache[:, :, hs].contiguous()), f(b.v_cache[:, :, hs].contiguous()), table

    per_head = [inputs(h) for h in heads]

    if path == "dcp":
        import oracle.dcp as odcp

    def run(a):
        if path == "dcp":
            odcp.dcp_chunked_prefill(*a, wl.block_size, wl.context_lens, sq, wl.workspace_rows, wl.split_alignment,
                                     wl.scale, dcp[0], dcp[1])
        else:
            fn = oracle.chunked_prefill if path == "chunked" else oracle.uniform_window_prefill
            fn(*a, wl.block_size, wl.context_lens, sq, wl.workspace_rows, wl.split_alignment, wl.scale)

    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, per_head))
        dt = time.perf_counter() - t0
    pairs = lambda ql: sum(a * c for a, c in zip(ql, wl.context_lens)) + sum(a * (a + 1) // 2 for a in ql)
    sample_flops = FLOP_PER_PAIR * len(heads) * pairs(sq)
    full_flops = FLOP_PER_PAIR * H * pairs(wl.query_lens)
    full = len(heads) == H and sq == list(wl.query_lens)
    what = (f"all {H} heads" if len(heads) == H else f"{len(heads)} of {H} heads (seeded)") + ", " + \
        ("all new tokens" if sample_queries is None else f"the first {sample_queries} new tokens of each request")
    return {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "seconds": round(dt, 3), "oracle_ms_per_step": round(dt * full_flops / sample_flops * 1e3, 1),
            "oracle_ms_kind": "measured" if full else "extrapolated",
            "machine_cpus": int(machine_cpus), "cpu_model": model,
            "sample": f"{what}, against full contexts (fp64 NumPy, whole {path} path); a pool of {workers} threads, "
                      f"one head per item, one BLAS thread each; value = sample flops / time"
                      + ("" if full else "; oracle_ms_per_step = time x full flops / sample flops")}


def mask_cpu_baseline(wl, heads=8):
    """The oracle's mask over all tokens of `heads` heads (fp64), repeated
    for about two seconds; value scaled to all heads as GB/s of the rows it
    writes."""
    import numpy as np
    import oracle
    ql, ctx = wl.query_lens, wl.context_lens
    qsl = np.concatenate([[0], np.cumsum(ql)])
    csl = np.concatenate([[0], np.cumsum(ctx)])
    T = wl.num_tokens
    lse = np.zeros((heads, T))
    out = np.zeros((T, heads, 128))
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.mask_empty_context(lse, out, qsl, csl)
        n += 1
        if time.perf_counter() - t0 > 2.0:
            break
    dt = (time.perf_counter() - t0) / n
    rows = sum(q for q, c in zip(ql, ctx) if c == 0)
    gbs = rows * wl.num_heads * (128 * 2 + 4) / (dt * wl.num_heads / heads) / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "seconds": round(dt * n, 3),
            "sample": f"{heads} of {wl.num_heads} heads, all {T} tokens, {n} repetitions (fp64 NumPy); time "
                      f"scaled by heads; bytes counted as the bf16 rows + fp32 LSE the kernel writes"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None,
                    choices=["tiny", "empty_context_stress", "homogeneous", "heterogeneous", "long_context", "skewed",
                             "heterogeneous_h16"],
                    help="default: long_context (chunked), heterogeneous (uniform_window, mask_empty_context)")
    ap.add_argument("--path", default="chunked", choices=["chunked", "uniform_window", "mask_empty_context", "dcp"])
    ap.add_argument("--dcp-world", type=int, default=4, help="emulated DCP ranks (--path dcp)")
    ap.add_argument("--dcp-interleave", type=int, default=1, help="DCP interleave run length (--path dcp)")
    ap.add_argument("--cpu-sample-queries", type=int, default=None,
                    help="oracle sample: first N new tokens of each request (default per workload)")
    ap.add_argument("--cpu-sample-heads", type=int, default=None, help="oracle sample: number of heads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload summary that the default run adds")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write profiles/<workload>_traffic.json from the counter collections of "
                         "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of this benchmark, then exit")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="after timing, run one elementwise copy (negation) of this many MiB of bf16 so that "
                         "hardware byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    # the default run (no --workload) also reports every named workload
    args.summary = args.workload is None and args.path == "chunked" and not args.no_workloads
    if args.workload is None:
        args.workload = "long_context" if args.path == "chunked" else "heterogeneous"
    return args


def timed_steps(mla, torch, step, steps, warmup):
    """W untimed steps, then K steps bracketed by device syncs, with every
    library kernel timed by HIP events on its own stream."""
    log(f"bench: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {steps} steps")
    mla.mla_kernel_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = mla.mla_kernel_timing_read()
    mla.mla_kernel_timing_enable(False)
    return (t1 - t0) / steps * 1e3, kt


KIND_WORK = {  # kernel kind -> (work figure, unit, bound)
    "chunk_attn": ("chunk_flops", "TFLOP/s", "mfma"), "suffix_attn": ("suffix_flops", "TFLOP/s", "mfma"),
    "gather": ("gather_bytes", "GB/s", "hbm"), "merge": ("merge_bytes", "GB/s", "hbm"),
    "mask": ("mask_bytes", "GB/s", "hbm"), "dcp_reorg": ("reorg_bytes", "GB/s", "hbm"),
    "init": (None, None, "hbm"),
}
KIND_KERNEL = {"chunk_attn": "chunk_attention_queued_kernel", "suffix_attn": "suffix_attention_queued_kernel",
               "gather": "gather_kernel", "merge": "merge_kernel_d128", "mask": "mask_empty_context_kernel",
               "dcp_reorg": "dcp_reorganize_kernel", "init": "init_partial_kernel"}


def kernel_table(kt, wf, K):
    kernels = {}
    for kind, (work, unit, _) in KIND_WORK.items():
        n, tms = kt[kind]
        if n == 0:
            continue
        e = {"launches_per_step": n / K, "ms_per_step": round(tms / K, 4)}
        if work is not None and tms > 0 and wf.get(work):
            rate = wf[work] * K / (tms / 1e3) / (1e12 if unit == "TFLOP/s" else 1e9)
            peak = PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
            e.update({"achieved": round(rate, 2), "unit": unit, "frac_of_peak": round(rate / peak, 4)})
        kernels[kind] = e
    return kernels


def roofline(kt, wf, K, workload, kind=None):
    """Roofline entry of the kernel kind with the most time (or `kind`)."""
    if kind is None:
        kind = max((k for k in KIND_WORK if KIND_WORK[k][0] is not None), key=lambda k: kt[k][1])
    work, unit, bound = KIND_WORK[kind]
    n, tms = kt[kind]
    per_launch = wf[work] * K / n if n else None
    achieved = wf[work] * K / (tms / 1e3) / (1e12 if unit == "TFLOP/s" else 1e9) if tms > 0 else None
    peak = PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
    r = {"kernel": kind, "bound": bound, "achieved": round(achieved, 2) if achieved else None, "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4) if achieved else None,
         "traffic": profiled_traffic(KIND_KERNEL[kind], workload),
         "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
         "launches_per_step": n / K, "avg_launch_ms": round(tms / n, 4) if n else None}
    if unit == "TFLOP/s":
        r["flops_per_launch"] = per_launch
        if kind == "chunk_attn":
            r["algorithmic_bytes_per_launch"] = wf["chunk_bytes"] * K / n if n else None
    else:
        r["algorithmic_bytes_per_launch"] = per_launch
    return r


def workload_summary(mla, torch, W, args, res):
    """Every named workload on the chunked path: step latency and kernel
    rates (10 timed steps after 2 warm-ups) beside the oracle's time for the
    same step on the host cores."""
    out = {}
    dev = "cuda:0"
    for idx, wl in W.named_workloads().items():
        if wl.name == args.workload:
            e = {"ms_per_step": res["ms_per_step"], "kernels": res["kernels"]}
            if "cpu_baseline" in res:
                e["cpu_oracle"] = res["cpu_baseline"]
            out[wl.name] = e
            continue
        log(f"bench: summary of {wl.name}")
        b = W.make_batch(wl, device=dev, canary=False)
        T, H = wl.num_tokens, wl.num_heads
        o = torch.empty((T, H, W.DV), dtype=torch.bfloat16, device=dev)
        l = torch.empty((H, T), dtype=torch.float32, device=dev)
        mk = lambda s=None: mla.make_prefill_params(  # noqa: E731
            b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens, wl.query_lens,
            wl.workspace_rows, wl.split_alignment, wl.scale, out=o, out_lse=l, scratch=s)
        scratch = torch.empty(max(256, mla.mla_chunked_prefill_scratch_size(mk())), dtype=torch.uint8, device=dev)
        p = mk(scratch)
        chunks, _, _ = mla.mla_plan_context_chunks(wl.context_lens, wl.query_lens, wl.workspace_rows, 0,
                                                   wl.split_alignment)
        ms, kt = timed_steps(mla, torch, lambda: mla.mla_chunked_prefill(p), 10, 2)
        e = {"ms_per_step": round(ms, 4), "kernels": kernel_table(kt, work_figures(wl, chunks), 10),
             "tokens": T, "context_rows": sum(wl.context_lens), "num_heads": H, "chunks": len(chunks)}
        del scratch
        if not args.no_cpu_baseline:
            log(f"bench: oracle on {wl.name}")
            e["cpu_oracle"] = cpu_baseline(b, wl)
        out[wl.name] = e
        del b, o, l
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: the chunked-prefill path here is single-GPU "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    import mla_chunked_context_amd as mla

    wl = W.workload_by_name(args.workload)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"bench: generating {wl.name} inputs on the GPU")
    b = W.make_batch(wl, device=dev, canary=False)
    T, H = wl.num_tokens, wl.num_heads
    K = args.steps
    out = torch.empty((T, H, W.DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    chunks, _, _ = mla.mla_plan_context_chunks(wl.context_lens, wl.query_lens, wl.workspace_rows, 0,
                                               wl.split_alignment)
    config = {"workload": wl.name, "num_requests": wl.num_requests, "query_lens": list(wl.query_lens),
              "context_lens": list(wl.context_lens), "num_heads": H, "qk_head_dim": 192, "v_head_dim": 128,
              "workspace_rows": wl.workspace_rows, "split_alignment": wl.split_alignment,
              "block_size": wl.block_size, "tokens": T, "context_rows": sum(wl.context_lens),
              "chunks": len(chunks), "continuation_chunks": sum(c["is_continuation"] for c in chunks),
              "value_std": wl.std, "path": args.path}

    def prefill_step(path, ranks=None):
        mk = lambda s=None: mla.make_prefill_params(  # noqa: E731
            b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens, wl.query_lens,
            wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse, scratch=s)
        if path == "dcp":
            scratch = torch.empty(mla.mla_dcp_chunked_prefill_scratch_size(mk(), ranks), dtype=torch.uint8,
                                  device=dev)
            p = mk(scratch)
            return (lambda: mla.mla_dcp_chunked_prefill(p, ranks)), scratch
        size = {"chunked": mla.mla_chunked_prefill_scratch_size,
                "uniform_window": mla.mla_uniform_window_prefill_scratch_size}[path]
        run = {"chunked": mla.mla_chunked_prefill, "uniform_window": mla.mla_uniform_window_prefill}[path]
        scratch = torch.empty(size(mk()), dtype=torch.uint8, device=dev)
        p = mk(scratch)
        return (lambda: run(p)), scratch

    extra = {}
    if args.path == "mask_empty_context":
        qsl = torch.tensor(np.concatenate([[0], np.cumsum(wl.query_lens)]), dtype=torch.int32, device=dev)
        csl = torch.tensor(np.concatenate([[0], np.cumsum(wl.context_lens)]), dtype=torch.int32, device=dev)
        lse.zero_()
        out.zero_()
        ms, kt = timed_steps(mla, torch, lambda: mla.mla_mask_empty_context(lse, out, qsl, csl), K, args.warmup)
        rows = sum(q for q, c in zip(wl.query_lens, wl.context_lens) if c == 0)
        wf = {"mask_bytes": rows * H * (128 * 2 + 4) + (wl.num_requests + 1) * 8}
        n, tms = kt["mask"]
        value = wf["mask_bytes"] * K / (tms / 1e3) / 1e9
        metric, unit = "mask_empty_context GB/s (rows written)", "GB/s"
        rf = roofline(kt, wf, K, wl.name, kind="mask")
        rf["masked_rows"] = rows
        kernels = kernel_table(kt, wf, K)
        steps_desc = "one mask launch over the batch"
    else:
        windows = None
        if args.path == "uniform_window":
            w, iters = mla.mla_plan_uniform_windows(wl.context_lens, wl.workspace_rows, wl.split_alignment)
            # rows of each request's window per iteration, for the work figures
            windows = [[max(0, min(c, (i + 1) * w) - i * w) for c in wl.context_lens] for i in range(iters)]
            config.update({"window": w, "iterations": iters})
        wf = work_figures(wl, chunks, windows)
        dranks = rank_caches = None
        if args.path == "dcp":
            D, il = args.dcp_world, args.dcp_interleave
            log(f"bench: sharding the context over {D} emulated ranks")
            rank_caches = W.shard_context(b, D, il, canary=False)
            dranks = mla.make_dcp_ranks(rank_caches, il)
            dch, *_ = mla.mla_plan_dcp_context_chunks(wl.context_lens, wl.query_lens, wl.workspace_rows, D, il, 0,
                                                      wl.split_alignment)
            # local gathers move every rank's padded rows; the reorganisation moves the context rows
            wf["gather_bytes"] = 2 * H * 640 * sum(c["num_rows"] for c in dch)
            wf["reorg_bytes"] = 2 * H * 640 * sum(wl.context_lens)
            config.update({"dcp_world": D, "dcp_interleave": il, "dcp_chunks": len(dch)})
        step, scratch = prefill_step(args.path, dranks)
        ms, kt = timed_steps(mla, torch, step, K, args.warmup)
        assert torch.isfinite(lse).all().item(), "non-finite LSE in the benchmark output"
        value = (wf["chunk_flops"] + wf["suffix_flops"]) / (ms / 1e3) / 1e12
        metric, unit = METRIC, "TFLOP/s"
        rf = roofline(kt, wf, K, wl.name)
        kernels = kernel_table(kt, wf, K)
        steps_desc = "the whole path over one batch"
        del scratch
        if args.path in ("uniform_window", "dcp"):
            step_c, scratch_c = prefill_step("chunked")
            ms_c, _ = timed_steps(mla, torch, step_c, K, args.warmup)
            del scratch_c
            if args.path == "uniform_window":
                extra["compare"] = {"uniform_window_ms_per_step": round(ms, 3), "chunked_ms_per_step": round(ms_c, 3),
                                    "chunked_speedup": round(ms / ms_c, 3), "iterations": config["iterations"],
                                    "chunks": len(chunks)}
            else:
                extra["compare"] = {"dcp_ms_per_step": round(ms, 3), "single_device_ms_per_step": round(ms_c, 3),
                                    "dcp_chunks": config["dcp_chunks"], "chunks": len(chunks)}

    res = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "step": steps_desc,
        "config": config, "roofline": rf, "kernels": kernels, **extra,
    }
    if args.calibration_copy_mb > 0:
        n = args.calibration_copy_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = {"read": n * 2, "write": n * 2}
        del src, dst
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle sample)")
        if args.path == "mask_empty_context":
            res["cpu_baseline"] = mask_cpu_baseline(wl)
        else:
            res["cpu_baseline"] = cpu_baseline(b, wl, args.path, rank_caches if args.path == "dcp" else None,
                                               (args.dcp_world, args.dcp_interleave), args.cpu_sample_heads,
                                               args.cpu_sample_queries)
    if args.summary:
        del b
        torch.cuda.empty_cache()
        res["workloads"] = workload_summary(mla, torch, W, args, res)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
