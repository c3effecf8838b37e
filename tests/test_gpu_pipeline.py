"""End-to-end parity of mla_chunked_prefill (the C ABI's whole path) with the
oracle.

* tiny and empty-context workloads, and random ragged ones: every output row
  and LSE against the oracle's chunked path (which the CPU tests pin to the
  direct definition), with NaN canaries in unused cache slots and scratch;
* 64- and 128-head batches (the wide-row gather and full head strides):
  every output row and LSE against the oracle;
* the full-size workloads, in the same launch configuration the benchmark
  times, with NaN canaries in unused cache slots: sampled rows (first, last,
  middle and random tokens of every request; a few heads) against the direct
  definition computed one row at a time, every row of every continuation
  request and every request without context for a seeded head, plus
  properties that hold at any size (no NaN, finite LSE everywhere).  Each
  check asserts the output's relative RMS error as well as its maximum.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import check, host, oracle_inputs, record, run_prefill, sampled_check, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"


def _full_case(wl):
    b = W.make_batch(wl, device="cpu", canary=True)
    ref = O.chunked_prefill(*oracle_inputs(b), wl.workspace_rows, wl.split_alignment, wl.scale)
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


# Chunk-attention launches whose longest workgroup outlasts the average CU load
# (work = heads x sum of query tiles x key tiles, over 256 CUs) cut each
# sequence's key range into slices and LSE-merge the slice states.  Each case's
# split count is the one with the shortest longest-first list schedule over
# the CUs (slices of at least 64 key tiles, at most 16; restated in
# tests/test_abi_host.py) and is given in the comment.
SPLIT_CASES = [
    # one chunk, 4 workgroups of 469 key tiles: 7 slices in one merge
    W.Workload("split_single", (30000,), (20,), 4, 32768, 64, 64, 1.0, 501),
    # 2 workgroups of 1024 key tiles: 16 slices, the most one merge combines
    W.Workload("split_sixteen", (65536,), (3,), 2, 65536, 64, 64, 1.0, 506),
    # chunk 0: request 0's first 16384 rows, 4 slices; chunk 1: its continuation
    # (13616 rows) in a launch of its own, 3 slices, then request 1's head
    W.Workload("split_continuation", (30000, 9000, 0), (5, 3, 2), 2, 16384, 64, 64, 1.0, 502),
    # three sequences in one launch, 4 slices of 5056 keys: the
    # shorter sequences' later slices are empty and merge as (0, -inf)
    W.Workload("split_ragged", (20000, 100, 5000), (4, 6, 2), 8, 32768, 64, 64, 1.0, 503),
    # a 16-head shard: 2 query tiles x 16 heads, 4 slices
    W.Workload("split_head_shard", (20000,), (300,), 16, 32768, 64, 64, 1.0, 504),
    # a request with no new tokens among split sequences: its workgroups exit
    # at once, the others' 4 slices merge as usual
    W.Workload("split_zero_query", (20000, 5000, 7000), (4, 0, 3), 4, 32768, 64, 64, 1.0, 505),
]


@pytest.mark.parametrize("wl", SPLIT_CASES, ids=[w.name for w in SPLIT_CASES])
def test_key_split_launches_match_oracle(wl):
    say(f"pipeline {wl.name} ctx={wl.context_lens} q={wl.query_lens} H={wl.num_heads} W={wl.workspace_rows}")
    res, *_ = _full_case(wl)
    say("  ", res)


# Wide head counts run the one-row-per-workgroup gather (at 52 heads and up)
# and the attention's 64- and 128-head strides; every row is checked.
WIDE_CASES = [
    # the tiny workload's lengths at 128 heads: two chunks, one continuation
    W.Workload("tiny_h128", (768, 512, 512, 0), (3, 5, 7, 4), 128, 1024, 64, 64, 1.0, 601),
    # 64 heads: request 0's context split over two chunks (chunk 0 holds its
    # first 8192 rows against 40 queries: 64 workgroups of 128 key tiles, so
    # the launch is cut into 2 key slices), a request without context, and a
    # last chunk of its own for request 3
    W.Workload("ragged_h64", (9000, 70, 0, 700), (40, 300, 5, 2), 64, 8192, 64, 64, 1.0, 602),
]


@pytest.mark.parametrize("wl", WIDE_CASES, ids=[w.name for w in WIDE_CASES])
def test_wide_head_workloads_full(wl):
    say(f"pipeline {wl.name} ctx={wl.context_lens} q={wl.query_lens} H={wl.num_heads} W={wl.workspace_rows}")
    res, *_ = _full_case(wl)
    record(f"chunked {wl.name} every row", res)


@pytest.mark.parametrize("rate", [0.3, -0.3, 0.03])
def test_suffix_pairs_with_rising_and_falling_scores(rate):
    # requests without context, so the prefill output is the causal suffix
    # alone: 700 and 1100 new tokens (3 and 5 query tiles: pairs (2, 0) and
    # (4, 0), (3, 1), a lone middle tile) whose scores rise (or fall) by about
    # rate * 40 log2 units per 64-key tile, so the running max of the tile
    # taken last-to-first moves the other way
    say(f"suffix pairs, score slope {rate}")
    g = torch.Generator().manual_seed(41)
    ql, H = (700, 1100), 2
    T = sum(ql)
    u = 2.0 * torch.randn(H, W.DK, generator=g)
    pos = torch.cat([torch.arange(n) for n in ql])
    q = (u[None] + torch.randn(T, H, W.DK, generator=g)).to(torch.bfloat16)
    k = ((pos // 64).float()[:, None, None] * rate * u[None] + torch.randn(T, H, W.DK, generator=g)).to(torch.bfloat16)
    v = torch.randn(T, H, W.DV, generator=g).to(torch.bfloat16)
    kc = torch.full((1, 64, H, W.DK), float("nan")).to(torch.bfloat16)
    vc = torch.full((1, 64, H, W.DV), float("nan")).to(torch.bfloat16)
    wl = W.Workload("suffix_pairs", (0, 0), ql, H, 256, 64, 64, 1.0, 0)
    bt = torch.zeros((2, 1), dtype=torch.int32)
    d = W.Batch(wl, q.to(DEV), k.to(DEV), v.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), 1)
    out, lse = run_prefill(mla, d)
    ref_o, ref_l = O.direct_prefill(host(q), host(k), host(v), host(kc), host(vc), bt.numpy(), 64, (0, 0), ql,
                                    wl.scale)
    record(f"suffix pairs slope {rate}", check(host(out), lse.double().cpu().numpy(), ref_o, ref_l,
                                               float(np.abs(host(v)).max()), f"slope {rate}"))


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


@pytest.mark.parametrize("name", ["split_continuation", "split_sixteen", "split_ragged"])
def test_queued_and_split_launches_are_repeatable(name):
    # which CU takes which item of a persistent launch changes from run to run
    # (per-XCD queues, stealing); each item's arithmetic and each merge's order
    # do not, so repeated runs agree bit for bit
    wl = [w for w in SPLIT_CASES if w.name == name][0]
    say(f"repeatability {name}")
    b = W.make_batch(wl, device=DEV, gen_device="cpu")
    o1, l1 = run_prefill(mla, b)
    for _ in range(3):
        o2, l2 = run_prefill(mla, b)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ------------------------------------------------------------- full sizes


@pytest.mark.timeout(600)
def test_homogeneous_full_size_sampled():
    sampled_check(mla, W.named_workloads()[3])


@pytest.mark.timeout(600)
def test_heterogeneous_full_size_sampled():
    sampled_check(mla, W.named_workloads()[4], tokens_per_request=4)


@pytest.mark.timeout(600)
def test_heterogeneous_h16_full_size_sampled():
    # one GPU's 16-head share: 7 of its 9 chunk-attention launches split keys
    sampled_check(mla, W.workload_by_name("heterogeneous_h16"), tokens_per_request=4)


@pytest.mark.timeout(600)
def test_long_context_full_size_sampled():
    sampled_check(mla, W.named_workloads()[5], tokens_per_request=8)


def test_side_stream_matches_default_stream():
    wl = W.named_workloads()[1]
    b = W.make_batch(wl, device=DEV, gen_device="cpu")
    o1, l1 = run_prefill(mla, b)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = run_prefill(mla, b, stream=s)
    s.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_many_calls_in_flight_reuse_staging_safely():
    # six calls enqueued without waiting (more than the pinned staging slots),
    # each on a different batch, must each equal its own call run alone
    say("six prefill calls in flight")
    cases = []
    for seed in range(6):
        wl = W.random_workload(100 + seed, max_requests=5, max_ctx=400, max_q=40, heads=(2,), alignments=(8, 16))
        cases.append(W.make_batch(wl, device=DEV, gen_device="cpu"))
    alone = [run_prefill(mla, b) for b in cases]
    outs = []
    for b in cases:
        wl = b.wl
        T, H = wl.num_tokens, wl.num_heads
        out = torch.full((T, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=DEV)
        mk = lambda s=None: mla.make_prefill_params(  # noqa: E731
            b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_table, wl.context_lens, wl.query_lens,
            wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse, scratch=s)
        scratch = torch.empty(max(256, mla.mla_chunked_prefill_scratch_size(mk())), dtype=torch.uint8, device=DEV)
        p = mk(scratch)
        mla.mla_chunked_prefill(p)  # no synchronisation between calls
        outs.append((out, lse, scratch, p))
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2, _, _) in zip(alone, outs):
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.timeout(600)
def test_skewed_full_size_sampled():
    sampled_check(mla, W.workload_by_name("skewed"), tokens_per_request=3)
