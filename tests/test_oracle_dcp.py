"""Pins of the oracle's DCP-local planning and context assembly (PR #50613
digest, 实现拆解 item 5 and 风险与影响; the sharding and padded_rows are
readings, see oracle/dcp.py).

* the position -> (rank, local index) rule is checked against brute-force
  enumeration of each rank's positions;
* padded_local is the most rows any rank holds, rounded up to whole runs;
* with one rank the plan is the single-device plan;
* plan invariants (exact coverage, all-gathered rows within the workspace,
  aligned splits);
* the reorganised all-gather equals the single-device gather, bit for bit;
* the whole DCP prefill equals the direct definition;
* a planted mistake in the local index is caught.
"""
import numpy as np
import pytest

import oracle as O
import oracle.dcp as D
import workloads as W

CASES = [(1, 1), (2, 1), (4, 1), (2, 2), (4, 4), (8, 1), (3, 2)]


@pytest.mark.parametrize("world,il", CASES)
def test_owner_and_local_index_enumerate_each_rank_in_order(world, il):
    for c in (0, 1, 7, il * world, 3 * il * world + 5, 257):
        held = [[] for _ in range(world)]
        for p in range(c):  # rank k % world holds run k = positions [k*il, (k+1)*il)
            held[(p // il) % world].append(p)
        for r in range(world):
            for li, p in enumerate(held[r]):
                assert D.dcp_owner(p, world, il) == r and D.dcp_local_index(p, world, il) == li
        assert [len(h) for h in held] == [D.local_context_lens([c], r, world, il)[0] for r in range(world)]


@pytest.mark.parametrize("world,il", CASES)
def test_padded_local_is_most_held_rounded_to_runs(world, il):
    for x in range(0, 200):
        most = max(D.local_context_lens([x], r, world, il)[0] for r in range(world))
        pad = D.padded_local_rows(x, world, il)
        assert most <= pad < most + il
        if il == 1 or x % (il * world) == 0:
            assert pad == most


def test_one_rank_is_the_single_device_plan():
    rng = np.random.default_rng(3)
    for _ in range(300):
        ctx = [0 if rng.random() < 0.2 else int(rng.integers(1, 900)) for _ in range(int(rng.integers(1, 9)))]
        a = int(rng.choice([1, 8, 64]))
        w = int(rng.integers(a, 2000))
        p1 = D.plan_dcp_context_chunks(ctx, w, a, 1, 1)
        p0 = O.plan_mla_context_chunks(ctx, w, None, a)
        assert [(p.request_start, p.request_end, p.starts, p.seq_lens) for p in p1] == \
            [(p.request_start, p.request_end, p.starts, p.seq_lens) for p in p0]


def test_plan_invariants_random():
    rng = np.random.default_rng(4)
    for _ in range(1500):
        world, il = CASES[int(rng.integers(0, len(CASES)))]
        a = world * il * int(rng.choice([1, 2, 4]))
        ctx = [0 if rng.random() < 0.2 else int(rng.integers(1, 1500)) for _ in range(int(rng.integers(1, 9)))]
        w = int(rng.integers(a, 3000))
        plans = D.plan_dcp_context_chunks(ctx, w, a, world, il)
        covered = [[] for _ in ctx]
        for pl in plans:
            _, lens, cu = D.dcp_local_entries(pl, world, il)
            assert world * int(cu[-1]) <= w
            for i, (s, n) in enumerate(zip(pl.starts, pl.seq_lens)):
                assert s % a == 0 and n > 0 and (i == 0 or s == 0)
                # every rank's positions of the entry fit its padded local rows
                for r in range(world):
                    held = [D.dcp_local_index(p, world, il) for p in range(s, s + n) if D.dcp_owner(p, world, il) == r]
                    assert all(s // world <= li < s // world + lens[i] for li in held)
                covered[pl.request_start + i].extend(range(s, s + n))
        assert [sorted(c) for c in covered] == [list(range(c)) for c in ctx]
    with pytest.raises(ValueError):
        D.plan_dcp_context_chunks([100], 256, 16, 4, 8)  # alignment not a multiple of world * interleave


@pytest.mark.parametrize("world,il", [(2, 1), (4, 1), (2, 4), (8, 2)])
def test_reorganised_all_gather_equals_single_device_gather(world, il):
    wl = W.Workload("dcp_small", (768, 300, 0, 515), (3, 5, 2, 4), 2, 512, 64, 16, 1.0, 8)
    b = W.make_batch(wl, canary=True)
    ranks = W.shard_context(b, world, il)
    kc = W.to_f64(b.k_cache)
    held = [rc.context_lens for rc in ranks]
    for pl in D.plan_dcp_context_chunks(wl.context_lens, wl.workspace_rows, wl.split_alignment, world, il):
        req = list(range(pl.request_start, pl.request_end))
        ls, ln, cu = D.dcp_local_entries(pl, world, il)
        gathered = np.concatenate([D.gather_local_rows(W.to_f64(rc.k_cache), rc.block_table.numpy(), 16, req, ls,
                                                       ln, held[r]) for r, rc in enumerate(ranks)])
        got = D.reorganize(gathered, pl, cu, world, il)
        ref = O.gather_context_rows(kc, b.block_table.numpy(), 16, req, pl.starts, pl.seq_lens)
        assert not np.isnan(got).any() and np.array_equal(got, ref)


@pytest.mark.parametrize("world,il", [(2, 1), (4, 2)])
def test_dcp_prefill_equals_direct(world, il):
    for seed in range(8):
        wl = W.random_workload(seed, max_ctx=200, max_q=10, alignments=(world * il, 2 * world * il))
        b = W.make_batch(wl, canary=True)
        ranks = W.shard_context(b, world, il)
        f = W.to_f64
        r = D.dcp_chunked_prefill(f(b.q), f(b.k_new), f(b.v_new), [f(x.k_cache) for x in ranks],
                                  [f(x.v_cache) for x in ranks], [x.block_table.numpy() for x in ranks],
                                  wl.block_size, wl.context_lens, wl.query_lens,
                                  max(wl.workspace_rows, wl.split_alignment), wl.split_alignment, wl.scale, world, il)
        d_out, d_lse = O.direct_prefill(f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache),
                                        b.block_table.numpy(), wl.block_size, wl.context_lens, wl.query_lens,
                                        wl.scale)
        assert not np.isnan(r["out"]).any(), seed
        assert np.abs(r["out"] - d_out).max(initial=0) < 1e-10, seed
        fin = np.isfinite(d_lse)
        assert (np.isfinite(r["lse"]) == fin).all() and np.abs(r["lse"][fin] - d_lse[fin]).max(initial=0) < 1e-10


def test_planted_local_index_mistake_is_caught(monkeypatch):
    # a local index that ignores the interleave runs reorders rows
    world, il = 2, 4
    wl = W.Workload("dcp_small", (300,), (3,), 1, 512, 64, 16, 1.0, 9)
    b = W.make_batch(wl, canary=True)
    ranks = W.shard_context(b, world, il)
    monkeypatch.setattr(D, "dcp_local_index", lambda p, w, i: p // w)
    pl = D.plan_dcp_context_chunks(wl.context_lens, wl.workspace_rows, wl.split_alignment, world, il)[0]
    ls, ln, cu = D.dcp_local_entries(pl, world, il)
    gathered = np.concatenate([D.gather_local_rows(W.to_f64(rc.k_cache), rc.block_table.numpy(), 16, [0], ls, ln,
                                                   rc.context_lens) for rc in ranks])
    got = D.reorganize(gathered, pl, cu, world, il)
    ref = O.gather_context_rows(W.to_f64(b.k_cache), b.block_table.numpy(), 16, [0], pl.starts, pl.seq_lens)
    assert not np.array_equal(np.nan_to_num(got, nan=1e9), ref)
