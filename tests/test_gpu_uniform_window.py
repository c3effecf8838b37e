"""End-to-end parity of mla_uniform_window_prefill (the earlier equal-window
scheduler with the empty-context mask in its loop) with the oracle's
uniform-window path, which the CPU tests pin to the direct definition.

Small cases compare every row; the heterogeneous and homogeneous full-size
workloads (the ones the scheduler comparison is measured on) are checked on
sampled rows against the direct definition.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import check, host, oracle_inputs, run_prefill, sampled_check, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"


def _full_case(wl):
    b = W.make_batch(wl, device="cpu", canary=True)
    ref = O.uniform_window_prefill(*oracle_inputs(b), wl.workspace_rows, wl.split_alignment, wl.scale)
    d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
    out, lse = run_prefill(mla, d, path="uniform_window")
    vals = np.concatenate([host(b.v_new).ravel(), np.nan_to_num(host(b.v_cache), nan=0.0).ravel()])
    vmax = float(np.abs(vals).max())
    res = check(host(out), lse.double().cpu().numpy(), ref["out"], ref["lse"], vmax, wl.name)
    return res, ref


def test_tiny_three_iterations():
    # window 320 rows: three iterations, the last two with empty windows (masked)
    wl = W.named_workloads()[1]
    assert mla.mla_plan_uniform_windows(wl.context_lens, wl.workspace_rows, wl.split_alignment) == (320, 3)
    say("uniform window tiny")
    res, ref = _full_case(wl)
    assert ref["iterations"] == 3
    say("  ", res)


def test_empty_context_stress_unaligned_window():
    # 33 requests with context share 256 rows: 7-row windows with alignment 1
    wl = dataclasses.replace(W.named_workloads()[2], split_alignment=1)
    say("uniform window empty-context stress, alignment 1")
    res, ref = _full_case(wl)
    assert ref["window"] == 7
    say("  ", res)


def test_random_workloads_full():
    for seed in range(12):
        wl = W.random_workload(seed, max_requests=7, max_ctx=700, max_q=150, heads=(1, 2, 3),
                               alignments=(1, 8, 16, 64))
        n_ctx = sum(c > 0 for c in wl.context_lens)
        # many iterations: a workspace of 1..4 aligned windows per request
        rows = max(1, n_ctx) * wl.split_alignment * (1 + seed % 4)
        wl = dataclasses.replace(wl, workspace_rows=rows)
        say(f"uniform window random seed={seed} ctx={wl.context_lens} q={wl.query_lens} H={wl.num_heads} "
            f"W={rows} A={wl.split_alignment} B={wl.block_size}")
        res, ref = _full_case(wl)
        say("  ", res, "iterations", ref["iterations"])


def test_homogeneous_full_size_sampled():
    sampled_check(mla, W.named_workloads()[3], path="uniform_window")


def test_heterogeneous_full_size_sampled():
    sampled_check(mla, W.named_workloads()[4], tokens_per_request=4, path="uniform_window")


def test_skewed_full_size_sampled():
    # one 131072-row context among 63 short ones: 64 equal-window iterations
    sampled_check(mla, W.workload_by_name("skewed"), tokens_per_request=3, path="uniform_window")
