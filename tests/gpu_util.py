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

import workloads as W

OUT_TOL = 2e-2
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_prefill(mla, b, out_lse=True, stream=None):
    """Run mla_chunked_prefill on a Batch that lives on the GPU."""
    wl = b.wl
    T, H = wl.num_tokens, wl.num_heads
    out = torch.full((T, H, W.DV), float("nan"), dtype=torch.bfloat16, device=b.q.device)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=b.q.device) if out_lse else None
    p = mla.make_prefill_params(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse)
    nbytes = mla.mla_chunked_prefill_scratch_size(p)
    scratch = torch.full(((max(nbytes, 256) + 1) // 2,), float("nan"), dtype=torch.bfloat16, device=b.q.device)
    p = mla.make_prefill_params(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse,
                                scratch=scratch)
    mla.mla_chunked_prefill(p, stream=stream)
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
