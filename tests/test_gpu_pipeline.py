"""End-to-end parity of mla_chunked_prefill (the C ABI's whole path) with the
oracle.

* tiny and empty-context workloads, and random ragged ones: every output row
  and LSE against the oracle's chunked path (which the CPU tests pin to the
  direct definition), with NaN canaries in unused cache slots and scratch;
* the full-size workloads, in the same launch configuration the benchmark
  times: sampled rows (first, last, middle and random tokens of requests; a
  few heads) against the direct definition computed one row at a time, plus
  properties that hold at any size (no NaN, finite LSE everywhere).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import check, host, run_prefill, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"


def _oracle_inputs(b):
    f = W.to_f64
    return (f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache), b.block_table.numpy(),
            b.wl.block_size, b.wl.context_lens, b.wl.query_lens)


def _full_case(wl):
    b = W.make_batch(wl, device="cpu", canary=True)
    ref = O.chunked_prefill(*_oracle_inputs(b), wl.workspace_rows, wl.split_alignment, wl.scale)
    d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
    out, lse = run_prefill(mla, d)
    vals = np.concatenate([host(b.v_new).ravel(), np.nan_to_num(host(b.v_cache), nan=0.0).ravel()])
    vmax = float(np.abs(vals).max())
    return check(host(out), lse.double().cpu().numpy(), ref["out"], ref["lse"], vmax, wl.name), ref, out, lse


@pytest.mark.parametrize("idx", [1, 2])
def test_named_small_workloads_full(idx):
    wl = W.named_workloads()[idx]
    say(f"pipeline {wl.name}")
    res, ref, out, lse = _full_case(wl)
    say("  ", res)
    if idx == 2:
        # the 131 rows of the request without context equal the suffix alone
        sfx = ref["suffix_out"][33:164]
        assert np.abs(host(out)[33:164] - sfx).max() <= 2e-2 * 5


def test_random_workloads_full():
    for seed in range(16):
        wl = W.random_workload(seed, max_requests=7, max_ctx=700, max_q=150, heads=(1, 2, 3),
                               alignments=(1, 8, 16, 64))
        say(f"pipeline random seed={seed} ctx={wl.context_lens} q={wl.query_lens} H={wl.num_heads} "
            f"W={wl.workspace_rows} A={wl.split_alignment} B={wl.block_size}")
        res, *_ = _full_case(wl)
        say("  ", res)


def test_run_twice_is_bitwise_identical():
    wl = W.named_workloads()[1]
    b = W.make_batch(wl, device=DEV, gen_device="cpu")
    o1, l1 = run_prefill(mla, b)
    o2, l2 = run_prefill(mla, b)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ------------------------------------------------------------- full sizes


def _context_rows(b, r, heads):
    wl = b.wl
    c = wl.context_lens[r]
    nb = (c + wl.block_size - 1) // wl.block_size
    blocks = b.block_table[r, :nb].long()
    hs = torch.tensor(heads, device=b.k_cache.device)
    k = b.k_cache.index_select(0, blocks).index_select(2, hs).reshape(nb * wl.block_size, len(heads), W.DK)[:c]
    v = b.v_cache.index_select(0, blocks).index_select(2, hs).reshape(nb * wl.block_size, len(heads), W.DV)[:c]
    return host(k), host(v)


def _sampled_check(idx, requests=None, tokens_per_request=6, seed=0):
    wl = W.named_workloads()[idx]
    say(f"pipeline full size {wl.name}: N={wl.num_requests} T={wl.num_tokens} ctx={sum(wl.context_lens)}")
    b = W.make_batch(wl, device=DEV, canary=False)
    out, lse = run_prefill(mla, b)
    say("  ran; checking")
    assert not torch.isnan(out).any().item() and torch.isfinite(lse).all().item()
    rng = np.random.default_rng(seed)
    H = wl.num_heads
    heads = sorted({0, H - 1, int(rng.integers(0, H)), int(rng.integers(0, H))})
    qsl = np.concatenate([[0], np.cumsum(wl.query_lens)])
    reqs = range(wl.num_requests) if requests is None else requests
    worst = {"out_err_over_vmax": 0.0, "lse_err": 0.0}
    hs = torch.tensor(heads, device=DEV)
    for r in reqs:
        n = wl.query_lens[r]
        if n == 0:
            continue
        pos = sorted({0, n - 1, n // 2, *[int(x) for x in rng.integers(0, n, size=max(0, tokens_per_request - 3))]})
        kc, vc = _context_rows(b, r, heads)
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


def test_homogeneous_full_size_sampled():
    _sampled_check(3)


def test_heterogeneous_full_size_sampled():
    _sampled_check(4, tokens_per_request=4)


def test_long_context_full_size_sampled():
    _sampled_check(5, tokens_per_request=8)
