"""Helpers of the GPU parity tests: running the library on a batch and the
tolerance checks against the oracle.

Tolerances (the pages give none; these are the bars set for this path):
  outputs  max |gpu - oracle| / max |V| <= 2e-2   (bf16 outputs)
           rms(gpu - oracle) / rms(oracle) <= 2e-2 over the checked rows
  LSE      max |gpu - oracle| <= 1e-3 on finite rows; -inf exactly where the
           oracle has -inf; no NaN anywhere.

The relative RMS bar is the sharp one on long contexts.  With 10^5 keys of
iid values, attention over a wrong set of keys still lands within the max
and LSE bars (the output is small against max |V| and the LSE is about
ln(n) + const), but its RMS error relative to the output is about 1.  The
GPU's own error is a few bf16 roundings (P, the output, each merge: 2^-9
relative each), about 5e-3 of the output's RMS.

When MLA_PARITY_LOG names a file, every checked case appends its error
figures to it as a JSON line, so the margins of a run are on record.
"""
import json
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O
import workloads as W

OUT_TOL = 2e-2
RMS_TOL = 2e-2
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def record(case, figures):
    """Print a case's error figures and append them to $MLA_PARITY_LOG."""
    say(f"  parity {case}: {figures}")
    path = os.environ.get("MLA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": case, **figures}) + "\n")


def run_prefill(mla, b, out_lse=True, stream=None, path="chunked"):
    """Run the whole path (mla_chunked_prefill, or mla_uniform_window_prefill
    with path="uniform_window") on a Batch that lives on the GPU."""
    size = {"chunked": mla.mla_chunked_prefill_scratch_size,
            "uniform_window": mla.mla_uniform_window_prefill_scratch_size}[path]
    run = {"chunked": mla.mla_chunked_prefill, "uniform_window": mla.mla_uniform_window_prefill}[path]
    wl = b.wl
    T, H = wl.num_tokens, wl.num_heads
    out = torch.full((T, H, W.DV), float("nan"), dtype=torch.bfloat16, device=b.q.device)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=b.q.device) if out_lse else None
    p = mla.make_prefill_params(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse)
    nbytes = size(p)
    scratch = torch.full(((max(nbytes, 256) + 1) // 2,), float("nan"), dtype=torch.bfloat16, device=b.q.device)
    p = mla.make_prefill_params(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse,
                                scratch=scratch)
    run(p, stream=stream)
    torch.cuda.synchronize()
    return out, lse


def run_dcp_prefill(mla, b, ranks, interleave):
    """Run mla_dcp_chunked_prefill on a Batch whose context lives in ``ranks``
    (RankCache list on the GPU, as workloads.shard_context makes them)."""
    wl = b.wl
    T, H = wl.num_tokens, wl.num_heads
    dev = b.q.device
    out = torch.full((T, H, W.DV), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev)
    dr = mla.make_dcp_ranks(ranks, interleave)

    def params(scratch=None):
        p = mla.make_prefill_params(b.q, b.k_new, b.v_new, None, None, None, wl.context_lens, wl.query_lens,
                                    wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse,
                                    scratch=scratch)
        p.block_size = wl.block_size
        return p

    n = mla.mla_dcp_chunked_prefill_scratch_size(params(), dr)
    scratch = torch.full(((max(n, 256) + 1) // 2,), float("nan"), dtype=torch.bfloat16, device=dev)
    mla.mla_dcp_chunked_prefill(params(scratch), dr)
    torch.cuda.synchronize()
    return out, lse


def host(t):
    return t.detach().float().cpu().double().numpy()


def check(out, lse, ref_out, ref_lse, vmax, what=""):
    """Assert the output/LSE bars; returns the error figures."""
    out = np.asarray(out, dtype=np.float64)
    ref_out = np.asarray(ref_out, dtype=np.float64)
    assert not np.isnan(out).any(), f"{what}: NaN in output"
    err = np.abs(out - ref_out).max(initial=0.0) / vmax
    rms = np.sqrt(np.mean((out - ref_out) ** 2)) / max(np.sqrt(np.mean(ref_out ** 2)), 1e-30) if out.size else 0.0
    res = {"out_err_over_vmax": float(err), "out_rel_rms": float(rms)}
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        ref_lse = np.asarray(ref_lse, dtype=np.float64)
        assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
        fin = np.isfinite(ref_lse)
        assert (np.isneginf(lse) == ~fin).all(), f"{what}: -inf pattern differs"
        lerr = np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0)
        res["lse_err"] = float(lerr)
        assert lerr <= LSE_TOL, f"{what}: LSE error {lerr}"
    assert err <= OUT_TOL, f"{what}: output error {err} x max|V|"
    assert rms <= RMS_TOL, f"{what}: output RMS error {rms} of the output's RMS"
    return res


def oracle_inputs(b):
    f = W.to_f64
    return (f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache), b.block_table.numpy(),
            b.wl.block_size, b.wl.context_lens, b.wl.query_lens)


def context_rows(b, r, heads):
    """Context rows 0..c-1 of request r, selected heads, read from the paged
    cache on the device (host float64 arrays)."""
    wl = b.wl
    c = wl.context_lens[r]
    nb = (c + wl.block_size - 1) // wl.block_size
    blocks = b.block_table[r, :nb].long()
    hs = torch.tensor(heads, device=b.k_cache.device)
    k = b.k_cache.index_select(0, blocks).index_select(2, hs).reshape(nb * wl.block_size, len(heads), W.DK)[:c]
    v = b.v_cache.index_select(0, blocks).index_select(2, hs).reshape(nb * wl.block_size, len(heads), W.DV)[:c]
    return host(k), host(v)


def continuation_requests(wl):
    """Requests whose context is split over chunks, from the oracle's plan:
    the first request of every chunk that starts past position 0."""
    plans = O.plan_mla_context_chunks(list(wl.context_lens), wl.workspace_rows, None, wl.split_alignment)
    return sorted({p.request_start for p in plans if p.starts and p.starts[0] > 0})


def _worst(into, res):
    for k, v in res.items():
        into[k] = max(into.get(k, 0.0), v)


def full_rows_check(b, out, lse, requests, heads, what):
    """Every row of ``requests`` for ``heads`` against the direct definition
    (oracle.direct_prefill, one thread per request)."""
    wl = b.wl
    if not requests:
        return {}
    hs = torch.tensor(heads, device=b.q.device)

    def sub(t, dim):
        return W.to_f64(t.index_select(dim, hs))
    q, kn, vn = sub(b.q, 1), sub(b.k_new, 1), sub(b.v_new, 1)
    kc, vc = sub(b.k_cache, 2), sub(b.v_cache, 2)
    table = b.block_table.cpu().numpy()
    qsl = np.concatenate([[0], np.cumsum(wl.query_lens)]).astype(np.int64)

    def one(r):
        return O.direct_prefill(q, kn, vn, kc, vc, table, wl.block_size, wl.context_lens, wl.query_lens, wl.scale,
                                requests=[r], query_block=256)
    with ThreadPoolExecutor(max_workers=min(8, len(requests))) as ex:
        refs = list(ex.map(one, requests))
    got_o = host(out.index_select(1, hs))
    got_l = lse.index_select(0, hs).double().cpu().numpy()
    worst = {}
    for r, (ref_o, ref_l) in zip(requests, refs):
        a, e = int(qsl[r]), int(qsl[r + 1])
        if a == e:
            continue
        c = wl.context_lens[r]
        nb = (c + wl.block_size - 1) // wl.block_size
        vrows = vc[table[r, :nb]].reshape(-1, len(heads), W.DV)[:c] if c else np.zeros((0,))
        vmax = float(max(np.abs(vrows).max(initial=0.0), np.abs(vn[a:e]).max(initial=0.0), 1e-30))
        _worst(worst, check(got_o[a:e], got_l[:, a:e], ref_o[a:e], ref_l[:, a:e], vmax, f"{what} request {r}"))
    return worst


def sampled_check(mla, wl, tokens_per_request=6, seed=0, path="chunked", device="cuda:0", runner=None,
                  full_row_heads=1):
    """Full-size run of a workload, with NaN canaries in every unused cache
    slot, checked against the direct definition:
      * sampled rows (first, last, middle and random tokens of each request)
        for a few heads, computed one row at a time;
      * every row of every continuation request and of every request without
        context, for ``full_row_heads`` seeded heads;
      * no NaN and a finite LSE everywhere.
    ``runner(batch) -> (out, lse)`` replaces run_prefill when given."""
    say(f"{path} full size {wl.name}: N={wl.num_requests} T={wl.num_tokens} ctx={sum(wl.context_lens)}")
    b = W.make_batch(wl, device=device, canary=True)
    out, lse = runner(b) if runner is not None else run_prefill(mla, b, path=path)
    say("  ran; checking")
    assert not torch.isnan(out).any().item() and torch.isfinite(lse).all().item()
    rng = np.random.default_rng(seed)
    H = wl.num_heads
    heads = sorted({0, H - 1, int(rng.integers(0, H)), int(rng.integers(0, H))})
    qsl = np.concatenate([[0], np.cumsum(wl.query_lens)])
    worst = {}
    hs = torch.tensor(heads, device=device)
    for r in range(wl.num_requests):
        n = wl.query_lens[r]
        if n == 0:
            continue
        pos = sorted({0, n - 1, n // 2, *[int(x) for x in rng.integers(0, n, size=max(0, tokens_per_request - 3))]})
        kc, vc = context_rows(b, r, heads)
        a = int(qsl[r])
        kn = host(b.k_new[a:a + max(pos) + 1].index_select(1, hs))
        vn = host(b.v_new[a:a + max(pos) + 1].index_select(1, hs))
        qr = host(b.q[[a + p for p in pos]].index_select(1, hs))
        ref_o, ref_l = O.direct_rows(qr, pos, kc, vc, kn, vn, wl.scale)
        got_o = host(out[[a + p for p in pos]].index_select(1, hs))
        got_l = lse.index_select(0, hs)[:, [a + p for p in pos]].double().cpu().numpy()
        vmax = float(max(np.abs(vc).max(initial=0), np.abs(vn).max()))
        _worst(worst, check(got_o, got_l, ref_o, ref_l, vmax, f"{wl.name} request {r}"))
    full = sorted(set(continuation_requests(wl)) | {r for r, c in enumerate(wl.context_lens) if c == 0})
    fheads = sorted({int(x) for x in rng.integers(0, H, size=full_row_heads)})
    say(f"  every row of requests {full} at heads {fheads}")
    fw = full_rows_check(b, out, lse, full, fheads, wl.name)
    record(f"{path} {wl.name} sampled rows, heads {heads}", worst)
    if fw:
        record(f"{path} {wl.name} every row of requests {full}, heads {fheads}", fw)
    del b, out, lse
    torch.cuda.empty_cache()
    return worst
