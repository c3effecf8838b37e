#!/usr/bin/env python3
"""Benchmark of MLA chunked-context prefill on one MI355X.

One step = the whole hot path over one batch: host planning and the metadata
upload, then per chunk gather -> chunk attention -> accumulate, the causal
suffix attention and the final merge (mla_chunked_prefill).  Inputs are
synthetic and already resident in HBM when the timed region starts.

Prints one JSON line.  `value` is the whole step's attention throughput:
algorithmic flops of chunk + suffix attention per second (2*(192+128) flops
per unmasked (query, key, head)).  `roofline` is for the dominant kernel
(chunk attention), timed live with HIP events on its own stream over the
timed region.  `cpu_baseline` times the fp64 oracle on a bounded sample of
the same workload on the host cores.
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


def work_figures(wl, chunks):
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
    # chunk attention must read Q, the gathered K/V rows and write O + LSE
    q_rows = sum(sum(ql[c["request_begin"]:c["request_end"]]) for c in chunks)
    chunk_bytes = H * (q_rows * (192 * 2 + 128 * 2 + 4) + rows * (192 + 128) * 2)
    return dict(chunk_flops=chunk_flops, suffix_flops=suffix_flops, gather_bytes=gather_bytes, chunk_bytes=chunk_bytes,
                merge_bytes=final_merge_bytes + accumulate_bytes, final_merge_bytes=final_merge_bytes,
                accumulate_bytes=accumulate_bytes)


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


def cpu_baseline(b, wl, sample_queries):
    """The oracle on a bounded sample: head 0 only and the first
    `sample_queries` new tokens of every request, against full contexts."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    qsl = np.concatenate([[0], np.cumsum(wl.query_lens)])
    sq = [min(sample_queries, q) for q in wl.query_lens]
    idx = np.concatenate([np.arange(qsl[r], qsl[r] + sq[r]) for r in range(wl.num_requests)]).astype(np.int64)
    it = torch.from_numpy(idx).to(b.q.device)
    f = W.to_f64
    q = f(b.q.index_select(0, it)[:, 0:1].contiguous())
    kn = f(b.k_new.index_select(0, it)[:, 0:1].contiguous())
    vn = f(b.v_new.index_select(0, it)[:, 0:1].contiguous())
    kc = f(b.k_cache[:, :, 0:1].contiguous())
    vc = f(b.v_cache[:, :, 0:1].contiguous())
    bt = b.block_table.cpu().numpy()
    t0 = time.perf_counter()
    oracle.chunked_prefill(q, kn, vn, kc, vc, bt, wl.block_size, wl.context_lens, sq, wl.workspace_rows,
                           wl.split_alignment, wl.scale)
    dt = time.perf_counter() - t0
    flops = FLOP_PER_PAIR * (sum(a * c for a, c in zip(sq, wl.context_lens)) + sum(a * (a + 1) // 2 for a in sq))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"head 0 of {wl.num_heads}, first {sample_queries} new tokens of each of the "
                      f"{wl.num_requests} requests against their full contexts (fp64 NumPy, whole chunked "
                      f"path: plan, gather, chunk attention, merges, causal suffix); value = sample flops / time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long_context",
                    choices=["tiny", "empty_context_stress", "homogeneous", "heterogeneous", "long_context"])
    ap.add_argument("--cpu-sample-queries", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="after timing, run one elementwise copy (negation) of this many MiB of bf16 so that "
                         "hardware byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: the chunked-prefill path here is single-GPU "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import mla_chunked_context_amd as mla

    wl = next(w for w in W.named_workloads().values() if w.name == args.workload)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"bench: generating {wl.name} inputs on the GPU")
    b = W.make_batch(wl, device=dev, canary=False)
    T, H = wl.num_tokens, wl.num_heads
    out = torch.empty((T, H, W.DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    p = mla.make_prefill_params(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse)
    scratch = torch.empty(mla.mla_chunked_prefill_scratch_size(p), dtype=torch.uint8, device=dev)
    p = mla.make_prefill_params(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse,
                                scratch=scratch)
    chunks, _, _ = mla.mla_plan_context_chunks(wl.context_lens, wl.query_lens, wl.workspace_rows, 0,
                                               wl.split_alignment)
    wf = work_figures(wl, chunks)
    stream = torch.cuda.current_stream()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        mla.mla_chunked_prefill(p)
    torch.cuda.synchronize()

    log(f"bench: timing {args.steps} steps")
    mla.mla_kernel_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mla.mla_chunked_prefill(p)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = mla.mla_kernel_timing_read()
    mla.mla_kernel_timing_enable(False)
    assert torch.isfinite(lse).all().item(), "non-finite LSE in the benchmark output"

    K = args.steps
    ms = (t1 - t0) / K * 1e3
    value = (wf["chunk_flops"] + wf["suffix_flops"]) / (ms / 1e3) / 1e12
    n_ca, ms_ca = kt["chunk_attn"]
    ca_tflops = wf["chunk_flops"] * K / (ms_ca / 1e3) / 1e12 if ms_ca > 0 else None
    kernels = {}
    for kind, work, unit in (("chunk_attn", wf["chunk_flops"], "TFLOP/s"),
                             ("suffix_attn", wf["suffix_flops"], "TFLOP/s"),
                             ("gather", wf["gather_bytes"], "GB/s"), ("merge", wf["merge_bytes"], "GB/s"),
                             ("init", None, None)):
        n, tms = kt[kind]
        e = {"launches_per_step": n / K, "ms_per_step": round(tms / K, 4)}
        if work is not None and tms > 0:
            rate = work * K / (tms / 1e3) / (1e12 if unit == "TFLOP/s" else 1e9)
            peak = PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
            e.update({"achieved": round(rate, 2), "unit": unit, "frac_of_peak": round(rate / peak, 4)})
        kernels[kind] = e

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "num_requests": wl.num_requests, "query_lens": list(wl.query_lens),
                   "context_lens": list(wl.context_lens), "num_heads": H, "qk_head_dim": 192, "v_head_dim": 128,
                   "workspace_rows": wl.workspace_rows, "split_alignment": wl.split_alignment,
                   "block_size": wl.block_size, "tokens": T, "context_rows": sum(wl.context_lens),
                   "chunks": len(chunks), "continuation_chunks": sum(c["is_continuation"] for c in chunks),
                   "value_std": wl.std},
        "roofline": {"kernel": "chunk_attn", "bound": "mfma",
                     "achieved": round(ca_tflops, 2) if ca_tflops else None, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ca_tflops / PEAK_BF16_TFLOPS, 4) if ca_tflops else None,
                     "traffic": profiled_traffic("chunk_attention_kernel", wl.name),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": (wf["chunk_bytes"] / n_ca * K) if n_ca else None,
                     "launches_per_step": n_ca / K,
                     "flops_per_launch": wf["chunk_flops"] * K / n_ca if n_ca else None,
                     "avg_launch_ms": round(ms_ca / n_ca, 4) if n_ca else None},
        "kernels": kernels,
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
    del scratch
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle sample)")
        res["cpu_baseline"] = cpu_baseline(b, wl, args.cpu_sample_queries)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
