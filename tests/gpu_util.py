"""Helpers of the GPU parity tests: running the library on a batch and the
tolerance checks against the oracle.

Tolerances (the pages give none; these are the bars set for this path):
  outputs  max |gpu - oracle| / max |V| <= 2e-2   (bf16 outputs)
  LSE      max |gpu - oracle| <= 1e-3 on finite rows; -inf exactly where the
           oracle has -inf; no NaN anywhere.
"""
import sys

import numpy as np
import torch

import oracle as O
import workloads as W

OUT_TOL = 2e-2
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


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


def sampled_check(mla, wl, tokens_per_request=6, seed=0, path="chunked", device="cuda:0", runner=None):
    """Full-size run of a workload, checked on sampled rows (first, last,
    middle and random tokens of each request; a few heads) against the direct
    definition computed one row at a time, plus no-NaN / finite-LSE everywhere.
    ``runner(batch) -> (out, lse)`` replaces run_prefill when given."""
    say(f"{path} full size {wl.name}: N={wl.num_requests} T={wl.num_tokens} ctx={sum(wl.context_lens)}")
    b = W.make_batch(wl, device=device, canary=False)
    out, lse = runner(b) if runner is not None else run_prefill(mla, b, path=path)
    say("  ran; checking")
    assert not torch.isnan(out).any().item() and torch.isfinite(lse).all().item()
    rng = np.random.default_rng(seed)
    H = wl.num_heads
    heads = sorted({0, H - 1, int(rng.integers(0, H)), int(rng.integers(0, H))})
    qsl = np.concatenate([[0], np.cumsum(wl.query_lens)])
    worst = {"out_err_over_vmax": 0.0, "lse_err": 0.0}
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
        res = check(got_o, got_l, ref_o, ref_l, vmax, f"{wl.name} request {r}")
        for k in worst:
            worst[k] = max(worst[k], res[k])
    say("  worst", worst)
    del b, out, lse
    torch.cuda.empty_cache()
    return worst
