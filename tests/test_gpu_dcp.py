"""GPU parity of the DCP pieces against the oracle, through the C ABI.

* mla_dcp_reorganize_context: per-rank local gathers (mla_gather_context on
  each rank's cache, written where an all-gather would put them), then the
  reorganisation, must equal the oracle's gather of the unsharded cache bit
  for bit, for every chunk of the plan;
* mla_dcp_chunked_prefill: every row and LSE against the oracle's DCP path on
  small and random batches, and sampled rows against the direct definition on
  the homogeneous batch sharded over 4 ranks.
"""
import numpy as np
import pytest
import torch

import oracle as O
import oracle.dcp as OD
import workloads as W
from tests.gpu_util import check, host, record, run_dcp_prefill, sampled_check, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"
SMALL = W.Workload("dcp_small", (768, 300, 0, 515, 64), (3, 5, 2, 4, 1), 2, 512, 64, 16, 1.0, 8)


def _i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)


@pytest.mark.parametrize("world,il", [(2, 1), (4, 1), (2, 4), (8, 2)])
def test_reorganize_equals_single_device_gather(world, il):
    wl = SMALL
    say(f"dcp reorganize world={world} interleave={il}")
    b = W.make_batch(wl, device="cpu", canary=True)
    ranks = W.shard_context(b, world, il)
    dranks = [W.RankCache(r.k_cache.to(DEV), r.v_cache.to(DEV), r.block_table.to(DEV), r.num_blocks, r.context_lens)
              for r in ranks]
    chunks, st, ln, lst, lln = mla.mla_plan_dcp_context_chunks(wl.context_lens, wl.query_lens, wl.workspace_rows,
                                                               world, il, 0, wl.split_alignment)
    H = wl.num_heads
    kc, vc = W.to_f64(b.k_cache), W.to_f64(b.v_cache)
    for c in chunks:
        e0, ne = c["entry_begin"], c["num_entries"]
        req = list(range(c["request_begin"], c["request_end"]))
        lcu = np.concatenate([[0], np.cumsum(lln[e0:e0 + ne])])
        cu = np.concatenate([[0], np.cumsum(ln[e0:e0 + ne])])
        L = int(lcu[-1])
        assert world * L == c["num_rows"]
        gk = torch.full((world * L, H, W.DK), float("nan"), dtype=torch.bfloat16, device=DEV)
        gv = torch.full((world * L, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
        for r, rc in enumerate(dranks):
            mla.mla_gather_context(rc.k_cache, rc.v_cache, rc.block_table, _i32(req), _i32(lst[e0:e0 + ne]),
                                   _i32(lcu), L, gk[r * L:(r + 1) * L], gv[r * L:(r + 1) * L])
        rows = int(cu[-1])
        wk = torch.full((rows, H, W.DK), float("nan"), dtype=torch.bfloat16, device=DEV)
        wv = torch.full((rows, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
        mla.mla_dcp_reorganize_context(gk, gv, world, il, L, _i32(st[e0:e0 + ne]), _i32(cu), _i32(lcu), rows, wk, wv)
        torch.cuda.synchronize()
        ref_k = O.gather_context_rows(kc, b.block_table.numpy(), wl.block_size, req, st[e0:e0 + ne], ln[e0:e0 + ne])
        ref_v = O.gather_context_rows(vc, b.block_table.numpy(), wl.block_size, req, st[e0:e0 + ne], ln[e0:e0 + ne])
        assert np.array_equal(host(wk), ref_k) and np.array_equal(host(wv), ref_v)


@pytest.mark.parametrize("world,il", [(2, 1), (4, 1), (4, 2)])
def test_dcp_prefill_small_full(world, il):
    wl = SMALL
    say(f"dcp prefill small world={world} interleave={il}")
    b = W.make_batch(wl, device="cpu", canary=True)
    ranks = W.shard_context(b, world, il)
    f = W.to_f64
    ref = OD.dcp_chunked_prefill(f(b.q), f(b.k_new), f(b.v_new), [f(r.k_cache) for r in ranks],
                                 [f(r.v_cache) for r in ranks], [r.block_table.numpy() for r in ranks], wl.block_size,
                                 wl.context_lens, wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale,
                                 world, il)
    d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
    dr = [W.RankCache(r.k_cache.to(DEV), r.v_cache.to(DEV), r.block_table.to(DEV), r.num_blocks, r.context_lens)
          for r in ranks]
    out, lse = run_dcp_prefill(mla, d, dr, il)
    vmax = float(max(np.abs(f(b.v_new)).max(), np.nanmax(np.abs(f(b.v_cache)))))
    say("  ", check(host(out), lse.double().cpu().numpy(), ref["out"], ref["lse"], vmax, "dcp small"))


def _random_with_context(count):
    """The first ``count`` seeded random DCP cases whose batch holds context
    (a batch without any exercises no rank assembly)."""
    seed = 0
    while count > 0:
        world, il = [(2, 1), (4, 1), (2, 2), (8, 1)][seed % 4]
        wl = W.random_workload(seed, max_requests=6, max_ctx=600, max_q=60, heads=(1, 2),
                               alignments=(world * il, 2 * world * il))
        seed += 1
        if sum(wl.context_lens) > 0:
            count -= 1
            yield seed - 1, world, il, wl


def test_dcp_prefill_random_full():
    for seed, world, il, wl in _random_with_context(8):
        say(f"dcp random seed={seed} world={world} il={il} ctx={wl.context_lens} q={wl.query_lens} "
            f"W={wl.workspace_rows} A={wl.split_alignment} B={wl.block_size}")
        b = W.make_batch(wl, device="cpu", canary=True)
        ranks = W.shard_context(b, world, il)
        f = W.to_f64
        ref = O.direct_prefill(f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache), b.block_table.numpy(),
                               wl.block_size, wl.context_lens, wl.query_lens, wl.scale)
        d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                    b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
        dr = [W.RankCache(r.k_cache.to(DEV), r.v_cache.to(DEV), r.block_table.to(DEV), r.num_blocks,
                          r.context_lens) for r in ranks]
        out, lse = run_dcp_prefill(mla, d, dr, il)
        vmax = float(max(np.abs(f(b.v_new)).max(), np.nanmax(np.abs(f(b.v_cache)))))
        say("  ", check(host(out), lse.double().cpu().numpy(), ref[0], ref[1], vmax, f"dcp random {seed}"))


def test_dcp_prefill_128_heads_full():
    # the small DCP batch at 128 heads: one-row gathers per rank, the
    # reorganisation and the attention at the full head stride, every row
    world, il = 4, 1
    wl = W.Workload("dcp_small_h128", SMALL.context_lens, SMALL.query_lens, 128, 512, 64, 16, 1.0, 10)
    say(f"dcp prefill {wl.name} world={world}")
    b = W.make_batch(wl, device="cpu", canary=True)
    ranks = W.shard_context(b, world, il)
    f = W.to_f64
    ref = OD.dcp_chunked_prefill(f(b.q), f(b.k_new), f(b.v_new), [f(r.k_cache) for r in ranks],
                                 [f(r.v_cache) for r in ranks], [r.block_table.numpy() for r in ranks], wl.block_size,
                                 wl.context_lens, wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale,
                                 world, il)
    d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
    dr = [W.RankCache(r.k_cache.to(DEV), r.v_cache.to(DEV), r.block_table.to(DEV), r.num_blocks, r.context_lens)
          for r in ranks]
    out, lse = run_dcp_prefill(mla, d, dr, il)
    vmax = float(max(np.abs(f(b.v_new)).max(), np.nanmax(np.abs(f(b.v_cache)))))
    record(f"dcp {wl.name} every row", check(host(out), lse.double().cpu().numpy(), ref["out"], ref["lse"], vmax,
                                             wl.name))


def test_dcp_prefill_with_key_split():
    # chunk 0 holds 16384 rows of request 0 against 10 queries at 2 heads: its
    # attention launch is cut into 4 key slices after the rows are assembled
    # from the 4 ranks
    world, il = 4, 1
    wl = W.Workload("dcp_split", (20000, 3000), (10, 4), 2, 16384, 64, 16, 1.0, 9)
    say(f"dcp key split world={world} ctx={wl.context_lens} q={wl.query_lens}")
    b = W.make_batch(wl, device="cpu", canary=True)
    ranks = W.shard_context(b, world, il)
    f = W.to_f64
    ref = O.direct_prefill(f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache), b.block_table.numpy(),
                           wl.block_size, wl.context_lens, wl.query_lens, wl.scale)
    d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
    dr = [W.RankCache(r.k_cache.to(DEV), r.v_cache.to(DEV), r.block_table.to(DEV), r.num_blocks, r.context_lens)
          for r in ranks]
    out, lse = run_dcp_prefill(mla, d, dr, il)
    vmax = float(max(np.abs(f(b.v_new)).max(), np.nanmax(np.abs(f(b.v_cache)))))
    say("  ", check(host(out), lse.double().cpu().numpy(), ref[0], ref[1], vmax, "dcp key split"))


@pytest.mark.timeout(600)
def test_dcp_homogeneous_full_size_sampled():
    world, il = 4, 1

    def runner(b):
        ranks = W.shard_context(b, world, il, canary=False)
        res = run_dcp_prefill(mla, b, ranks, il)
        del ranks
        return res

    sampled_check(mla, W.named_workloads()[3], path=f"dcp world={world}", runner=runner)


def test_reorganize_inconsistent_metadata_writes_nan_rows():
    # local_rows too small for the entry: rows whose source falls past the
    # gathered buffer come out NaN; every other row is a copy (no fault)
    say("dcp reorganize with inconsistent local_rows")
    H, world, L = 1, 2, 2
    gk = torch.arange(world * L * H * W.DK, dtype=torch.float32).reshape(world * L, H, W.DK).to(torch.bfloat16)
    gv = torch.arange(world * L * H * W.DV, dtype=torch.float32).reshape(world * L, H, W.DV).to(torch.bfloat16)
    gk, gv = gk.to(DEV), gv.to(DEV)
    wk = torch.zeros((8, H, W.DK), dtype=torch.bfloat16, device=DEV)
    wv = torch.zeros((8, H, W.DV), dtype=torch.bfloat16, device=DEV)
    mla.mla_dcp_reorganize_context(gk, gv, world, 1, L, _i32([0]), _i32([0, 8]), _i32([0, 2]), 8, wk, wv)
    torch.cuda.synchronize()
    k, gkh = host(wk), host(gk)
    for p in range(8):
        src = (p % 2) * L + p // 2
        if src >= world * L:
            assert np.isnan(k[p]).all(), p
        else:
            assert np.array_equal(k[p], gkh[src]), p
