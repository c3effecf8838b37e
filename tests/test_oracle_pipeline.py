"""Pins of the oracle's chunked path: it must equal the direct definition
(one softmax per token over its request's context and causal new tokens) on
tiny inputs, leave requests without context at (0, -inf) in the partial, and
never let NaN canaries from unused cache slots through.  A last group plants
plausible mistakes in the oracle and checks that these pins catch them.
"""
import numpy as np
import pytest

import oracle as O
import oracle.merge as OM
import oracle.pipeline as OP
import oracle.planner as OPL
import workloads as W


def _arrays(b):
    f = W.to_f64
    return (f(b.q), f(b.k_new), f(b.v_new), f(b.k_cache), f(b.v_cache), b.block_table.numpy(),
            b.wl.block_size, b.wl.context_lens, b.wl.query_lens)


def _both(wl):
    b = W.make_batch(wl, canary=True)
    a = _arrays(b)
    r = O.chunked_prefill(*a, wl.workspace_rows, wl.split_alignment, wl.scale)
    d = O.direct_prefill(*a, wl.scale)
    return r, d


@pytest.mark.parametrize("idx", [1, 2])
def test_chunked_equals_direct_named(idx):
    r, (d_out, d_lse) = _both(W.named_workloads()[idx])
    assert not np.isnan(r["out"]).any() and not np.isnan(r["lse"]).any()
    assert np.abs(r["out"] - d_out).max() < 1e-10
    assert np.abs(r["lse"] - d_lse).max() < 1e-10


def test_chunked_equals_direct_random():
    for seed in range(60):
        wl = W.random_workload(seed, max_ctx=120, max_q=12)
        r, (d_out, d_lse) = _both(wl)
        assert np.abs(r["out"] - d_out).max() < 1e-10, seed
        fin = np.isfinite(d_lse)
        assert (np.isfinite(r["lse"]) == fin).all(), seed
        assert np.abs(r["lse"][fin] - d_lse[fin]).max(initial=0) < 1e-10, seed


def test_empty_context_rows(golden):
    """PR #49294 digest, test_mask_empty_context: rows 33..163 belong to the
    request without context and end with LSE -inf and output 0 in the context
    partial; the final result of those rows is the suffix alone."""
    g = golden("empty_context_rows.json")
    wl = W.Workload("p1_empty_rows", tuple(g["context_lens"]), tuple(g["query_lens"]), g["num_heads"],
                    256, 16, 16, 1.0, 2)
    assert wl.num_tokens == g["num_tokens"]
    b = W.make_batch(wl, canary=True)
    r = O.chunked_prefill(*_arrays(b), wl.workspace_rows, wl.split_alignment, wl.scale)
    e0, e1 = g["empty_rows"]
    assert (r["partial_out"][e0:e1] == 0).all()
    assert np.isneginf(r["partial_lse"][:, e0:e1]).all()
    others = np.r_[0:e0, e1:g["num_tokens"]]
    assert np.isfinite(r["partial_lse"][:, others]).all()
    assert np.array_equal(r["out"][e0:e1], r["suffix_out"][e0:e1])
    assert np.array_equal(r["lse"][:, e0:e1], r["suffix_lse"][:, e0:e1])
    assert not np.isnan(r["out"]).any()


def test_fast_path_shape_single_chunk():
    # one chunk covering all tokens: the partial equals that chunk's attention
    wl = W.Workload("one_chunk", (100, 60), (4, 3), 2, 256, 16, 16, 1.0, 3)
    b = W.make_batch(wl)
    r = O.chunked_prefill(*_arrays(b), wl.workspace_rows, wl.split_alignment, wl.scale)
    assert len(r["metadata"].chunks) == 1 and r["metadata"].chunks[0].token_slice == (0, 7)


# ------------------------------------------------- planted mistakes


def _pins_pass():
    try:
        test_chunked_equals_direct_named(1)
        test_chunked_equals_direct_random()
        return True
    except AssertionError:
        return False


def test_pins_catch_overwrite_instead_of_merge(monkeypatch):
    def overwrite(p_out, p_lse, c_out, c_lse, token_slice):
        t0, t1 = token_slice
        p_out[t0:t1] = c_out
        p_lse[:, t0:t1] = c_lse
    monkeypatch.setattr(OP, "accumulate_mla_context_chunk", overwrite)
    assert not _pins_pass()


def test_pins_catch_gather_off_by_one(monkeypatch):
    real = OP.gather_context_rows

    def shifted(cache, table, bs, reqs, starts, lens):
        return real(cache, table, bs, reqs, [s + (1 if s > 0 else 0) for s in starts], lens)
    monkeypatch.setattr(OP, "gather_context_rows", shifted)
    assert not _pins_pass()


def test_pins_catch_wrong_merge_weight_sign(monkeypatch):
    real = OM.merge_states

    def bad(a_out, a_lse, b_out, b_lse):
        o, l = real(a_out, a_lse, b_out, b_lse)
        o2, _ = real(a_out, np.negative(a_lse), b_out, np.negative(b_lse))
        return o2, l
    monkeypatch.setattr(OM, "merge_states", bad)
    assert not _pins_pass()


def test_pins_catch_causal_off_by_one(monkeypatch):
    import oracle.attention as OA

    def strict(q, k, v, scale, q0):
        nq = q.shape[0]
        nk = q0 + nq
        s = scale * (q @ k[:nk].T)
        vis = np.arange(nk)[None, :] < np.maximum(1, q0 + np.arange(nq))[:, None]
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        return (e @ v[:nk]) / l, (m + np.log(l))[:, 0]
    monkeypatch.setattr(OA, "_attend_causal_block", strict)
    assert not _pins_pass()


def test_pins_catch_dropped_last_entry(monkeypatch):
    real = OPL.plan_mla_context_chunks

    def drop(*a, **k):
        plans = real(*a, **k)
        for p in plans:
            if len(p.seq_lens) > 1:
                p.seq_lens[-1] -= 1
        return plans
    monkeypatch.setattr(OP, "plan_mla_context_chunks", drop)
    assert not _pins_pass()


def test_pins_catch_missing_threshold(monkeypatch):
    """Without the threshold copy, a trailing request with no context would
    still be right (its partial is empty), so plant the opposite mistake:
    copying the suffix for every row."""
    real = OP.merge_attn_states
    monkeypatch.setattr(OP, "merge_attn_states", lambda po, pl, so, sl, k: real(po, pl, so, sl, 0))
    assert not _pins_pass()


def test_direct_prefill_query_blocks_only_bound_memory():
    # blocks of 3 tokens cut requests mid-way; every row is still the definition
    for seed in (1, 4, 7):
        wl = W.random_workload(seed, max_ctx=120, max_q=12)
        a = _arrays(W.make_batch(wl, canary=True))
        d_out, d_lse = O.direct_prefill(*a, wl.scale)
        b_out, b_lse = O.direct_prefill(*a, wl.scale, query_block=3)
        assert np.allclose(b_out, d_out, rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(b_lse), np.isneginf(d_lse))
        fin = np.isfinite(d_lse)
        assert np.allclose(b_lse[fin], d_lse[fin], rtol=0, atol=1e-12)


def test_direct_rows_matches_direct_prefill():
    wl = W.named_workloads()[1]
    b = W.make_batch(wl)
    a = _arrays(b)
    d_out, d_lse = O.direct_prefill(*a, wl.scale)
    f = W.to_f64
    # request 1: context 512 rows, 5 new tokens starting at token 3
    table = b.block_table.numpy()
    rows = [f(b.k_cache)[table[1][p // 64], p % 64] for p in range(512)]
    vrows = [f(b.v_cache)[table[1][p // 64], p % 64] for p in range(512)]
    out, lse = O.direct_rows(f(b.q)[[4, 7]], [1, 4], np.stack(rows), np.stack(vrows), f(b.k_new)[3:8],
                             f(b.v_new)[3:8], wl.scale)
    assert np.allclose(out, d_out[[4, 7]], atol=1e-13) and np.allclose(lse, d_lse[:, [4, 7]], atol=1e-13)


def test_mask_empty_context_printed_test(golden):
    """PR #49294 digest, test_mask_empty_context: random LSE/outputs with the
    empty request's rows NaN; afterwards those rows are (-inf, 0) and every
    other value is unchanged."""
    g = golden("empty_context_rows.json")
    H, T, D = g["num_heads"], g["num_tokens"], g["head_dim"]
    qsl = np.concatenate([[0], np.cumsum(g["query_lens"])])
    csl = np.concatenate([[0], np.cumsum(g["context_lens"])])
    rng = np.random.default_rng(0)
    lse = rng.standard_normal((H, T)).astype(np.float32)
    out = rng.standard_normal((T, H, D)).astype(np.float32)
    e0, e1 = g["empty_rows"]
    out[e0:e1] = np.nan
    exp_lse, exp_out = lse.copy(), out.copy()
    exp_lse[:, e0:e1] = -np.inf
    exp_out[e0:e1] = 0.0
    O.mask_empty_context(lse, out, qsl, csl)
    assert np.array_equal(lse, exp_lse) and np.array_equal(out, exp_out)


def test_mask_then_merge_equals_init_partial():
    """Both mechanisms give the same context partial: chunk results merged
    into an uninitialised partial after masking the empty rows equal the
    init-then-accumulate path."""
    wl = W.named_workloads()[2]
    b = W.make_batch(wl)
    r = O.chunked_prefill(*_arrays(b), wl.workspace_rows, wl.split_alignment, wl.scale)
    md = r["metadata"]
    # partial built the P1 way: start from garbage, every chunk writes its rows,
    # then rows of requests without context are masked
    out = np.full_like(r["partial_out"], np.nan)
    lse = np.full_like(r["partial_lse"], np.nan)
    for ch in md.chunks:
        t0, t1 = ch.token_slice
        out[t0:t1] = r["partial_out"][t0:t1]
        lse[:, t0:t1] = r["partial_lse"][:, t0:t1]
    csl = np.concatenate([[0], np.cumsum(wl.context_lens)])
    O.mask_empty_context(lse, out, md.query_start_loc, csl)
    assert np.array_equal(out, r["partial_out"]) and np.array_equal(lse, r["partial_lse"])
