"""Pins of the oracle's uniform-window scheduler (the scheduling per-request
packing replaced, PR #50613 digest, 功能与动机, with the PR #49294 digest's
empty-context mask in its loop).

The window rule is pinned by a hand derivation and by invariants; the
prefill result by the direct definition (one softmax per token), which it must
equal up to rounding; the mask step by planting its omission.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W


def _arrays(b):
    f = W.to_f64
    return (f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache), b.block_table.numpy(),
            b.wl.block_size, b.wl.context_lens, b.wl.query_lens)


def test_window_rule_by_hand():
    # ctx [768, 512, 512, 0], W = 1024, A = 64: three requests share the
    # workspace, 1024 // 3 = 341 rows each, 320 after aligning; 768 rows take
    # three windows: [0,320), [320,640), [640,768).
    w, starts, lens = O.plan_uniform_windows([768, 512, 512, 0], 1024, 64)
    assert w == 320
    assert starts == [[0] * 4, [320] * 4, [640] * 4]
    assert lens == [[320, 320, 320, 0], [320, 192, 192, 0], [128, 0, 0, 0]]
    # the unaligned share
    assert O.uniform_window_size([768, 512, 512, 0], 1024, 1) == 341


def test_window_rule_special_cases():
    assert O.plan_uniform_windows([0, 0], 64, 16) == (0, [], [])
    assert O.uniform_window_size([5], 64, 16) == 64  # one request takes the whole workspace
    with pytest.raises(ValueError):
        O.uniform_window_size([10, 10, 10], 40, 16)  # 13 rows each, no 16-row window
    with pytest.raises(ValueError):
        O.uniform_window_size([10], 0, 1)


def test_window_invariants_random():
    rng = np.random.default_rng(5)
    for _ in range(2000):
        n = int(rng.integers(1, 12))
        ctx = [0 if rng.random() < 0.3 else int(rng.integers(1, 3000)) for _ in range(n)]
        a = int(rng.choice([1, 4, 16, 64]))
        n_ctx = sum(c > 0 for c in ctx)
        W_ = int(rng.integers(max(1, n_ctx) * a, max(1, n_ctx) * a * 40 + 1))
        w, starts, lens = O.plan_uniform_windows(ctx, W_, a)
        if n_ctx == 0:
            assert (w, starts, lens) == (0, [], [])
            continue
        assert w % a == 0 and w >= a and w * n_ctx <= W_
        assert w + a > W_ // n_ctx  # the largest aligned window within the share
        assert len(lens) == math.ceil(max(ctx) / w)
        for it, row in enumerate(lens):
            assert sum(row) <= W_
            for r in range(n):
                assert starts[it][r] == it * w and 0 <= row[r] <= w
        # every context row is covered exactly once, windows in order
        for r in range(n):
            covered = [starts[it][r] + j for it in range(len(lens)) for j in range(lens[it][r])]
            assert covered == list(range(ctx[r]))


def _uw(wl, skip_mask=False):
    b = W.make_batch(wl, canary=True)
    a = _arrays(b)
    n_ctx = sum(c > 0 for c in wl.context_lens)
    rows = max(wl.workspace_rows, n_ctx * wl.split_alignment)
    r = O.uniform_window_prefill(*a, rows, wl.split_alignment, wl.scale, skip_mask=skip_mask)
    return r, O.direct_prefill(*a, wl.scale), a, rows


def test_uniform_window_equals_direct_tiny():
    wl = W.named_workloads()[1]
    r, (d_out, d_lse), _, _ = _uw(wl)
    assert r["window"] == 320 and r["iterations"] == 3
    assert not np.isnan(r["out"]).any() and not np.isnan(r["lse"]).any()
    assert np.abs(r["out"] - d_out).max() < 1e-10
    assert np.abs(r["lse"] - d_lse).max() < 1e-10


def test_uniform_window_equals_direct_random():
    for seed in range(40):
        wl = W.random_workload(seed, max_ctx=120, max_q=12)
        r, (d_out, d_lse), _, _ = _uw(wl)
        assert not np.isnan(r["out"]).any(), seed
        assert np.abs(r["out"] - d_out).max(initial=0) < 1e-10, seed
        fin = np.isfinite(d_lse)
        assert (np.isfinite(r["lse"]) == fin).all(), seed
        assert np.abs(r["lse"][fin] - d_lse[fin]).max(initial=0) < 1e-10, seed


def test_uniform_window_partial_matches_chunked_partial():
    # both schedulers compute the same context partial (up to rounding); rows
    # of requests without context are (0, -inf) exactly in both
    wl = W.named_workloads()[1]
    b = W.make_batch(wl, canary=True)
    a = _arrays(b)
    u = O.uniform_window_prefill(*a, wl.workspace_rows, wl.split_alignment, wl.scale)
    c = O.chunked_prefill(*a, wl.workspace_rows, wl.split_alignment, wl.scale)
    fin = np.isfinite(c["partial_lse"])
    assert (np.isfinite(u["partial_lse"]) == fin).all()
    assert np.abs(u["partial_lse"][fin] - c["partial_lse"][fin]).max() < 1e-10
    e0, e1 = 15, 19  # request 3 (no context)
    assert (u["partial_out"][e0:e1] == 0).all() and np.isneginf(u["partial_lse"][:, e0:e1]).all()


def test_planted_missing_mask_is_caught():
    # without the mask the unspecified result of empty windows reaches the merge
    wl = W.named_workloads()[1]
    r, (d_out, _), _, _ = _uw(wl, skip_mask=True)
    assert np.isnan(r["out"]).any() or np.abs(r["out"] - d_out).max() > 1e-6
