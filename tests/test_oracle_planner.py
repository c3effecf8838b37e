"""Pins of the oracle planner against what the pages fix.

* the printed worked example (PR #50613 digest, test_tail_splitting_minimizes_chunks);
* the packing invariants the digest states (实现拆解 item 2 and the test file
  description): every context row gathered exactly once, no chunk over the
  workspace, no request without context inside a chunk, continuation only in a
  chunk's first request, request order kept;
* minimality (the example's docstring: two chunks is the least possible under
  the row budget), checked against brute force over all valid aligned packings.
"""
import functools

import numpy as np
import pytest

import oracle as O
import workloads as W


def _plan(ctx, w, a, m=None):
    return O.plan_mla_context_chunks(ctx, w, m, a)


@pytest.mark.parametrize("alignment", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_printed_example(golden, alignment):
    g = golden("tail_split_example.json")
    md = O.build_chunked_context(g["context_lens"], g["query_lens"], g["workspace_rows"], split_alignment=alignment)
    assert len(md.chunks) == len(g["chunks"])
    for ch, exp in zip(md.chunks, g["chunks"]):
        assert ch.starts.tolist() == exp["starts"]
        assert ch.seq_lens.tolist() == exp["seq_lens"]
        assert ch.is_continuation == exp["is_continuation"]
    # the chunks' request slices follow from starts/seq_lens: (0,2) then (1,3)
    assert [c.request_slice for c in md.chunks] == [(0, 2), (1, 3)]
    assert [c.token_slice for c in md.chunks] == [(0, 8), (3, 15)]


def _check_invariants(ctx, w, a, m, plans):
    m = w if m is None else m
    covered = {r: [] for r in range(len(ctx))}
    prev_end = -1
    for p in plans:
        # a contiguous request slice, in order, never revisiting earlier requests
        assert p.request_end - p.request_start == len(p.starts) == len(p.seq_lens) >= 1
        assert p.request_start >= prev_end - 1
        prev_end = p.request_end
        assert sum(p.seq_lens) <= w, "chunk exceeds the workspace"
        assert p.is_continuation == (p.starts[0] > 0)
        for i, (s, n) in enumerate(zip(p.starts, p.seq_lens)):
            r = p.request_start + i
            assert ctx[r] > 0, "request without context inside a chunk"
            assert n > 0
            if i > 0:
                assert s == 0, "continuation outside a chunk's first request"
            if i < len(p.starts) - 1:
                assert s + n == ctx[r], "only the last entry of a chunk may stop early"
            assert s % a == 0, "split point off the alignment grid"
            if s + n < ctx[r]:
                assert n % a == 0 and n <= m, "a split piece must be aligned and capped"
            covered[r].append((s, n))
    for r, c in enumerate(ctx):
        pieces = sorted(covered[r])
        pos = 0
        for s, n in pieces:
            assert s == pos, "gap or overlap in a request's context rows"
            pos += n
        assert pos == c, "context rows not covered exactly once"


def test_invariants_random():
    for seed in range(3000):
        wl = W.random_workload(seed)
        m = None if seed % 3 else wl.workspace_rows // 2 if wl.workspace_rows // 2 >= wl.split_alignment else None
        plans = _plan(wl.context_lens, wl.workspace_rows, wl.split_alignment, m)
        _check_invariants(list(wl.context_lens), wl.workspace_rows, wl.split_alignment, m, plans)


def test_invariants_named_workloads():
    for i, wl in W.named_workloads().items():
        plans = _plan(wl.context_lens, wl.workspace_rows, wl.split_alignment)
        _check_invariants(list(wl.context_lens), wl.workspace_rows, wl.split_alignment, None, plans)


def _min_chunks_bruteforce(ctx, w, a, m):
    """Least number of chunks over every valid packing: chunks are contiguous
    request slices (never crossing a request without context), cut inside a
    request only at multiples of the alignment (piece length <= m), each
    holding at most w rows."""
    n = len(ctx)

    @functools.lru_cache(maxsize=None)
    def best(r, p):
        while r < n and ctx[r] == 0:
            r += 1
        if r == n:
            return 0
        result = None
        # enumerate every chunk that starts at (r, p)
        stack = [(r, p, 0)]  # (request, offset, rows used) inside the chunk being built
        while stack:
            rr, pp, used = stack.pop()
            rem = ctx[rr] - pp
            room = w - used
            # close the chunk after an aligned partial piece of request rr
            for length in range(a, min(rem - 1, m) + 1, a):
                if length <= room:
                    sub = best(rr, pp + length)
                    result = sub + 1 if result is None else min(result, sub + 1)
            if rem <= room:
                # take the whole remainder of rr, then close or continue
                sub = best(rr + 1, 0)
                result = sub + 1 if result is None else min(result, sub + 1)
                if rr + 1 < n and ctx[rr + 1] > 0:
                    stack.append((rr + 1, 0, used + rem))
        assert result is not None
        return result

    return best(0, 0)


def test_minimal_chunk_count_bruteforce():
    rng = np.random.default_rng(123)
    checked = 0
    for _ in range(1500):
        n = int(rng.integers(1, 6))
        a = int(rng.choice([1, 2, 4, 8]))
        ctx = [0 if rng.random() < 0.2 else int(rng.integers(1, 40)) for _ in range(n)]
        w = int(rng.integers(a, 48))
        m = w if rng.random() < 0.7 else int(rng.integers(a, w + 1))
        plans = _plan(ctx, w, a, m)
        assert len(plans) == _min_chunks_bruteforce(tuple(ctx), w, a, m), (ctx, w, a, m)
        checked += 1
    assert checked == 1500


def test_aligned_split_len_values():
    # hand-computed from the definition: the largest multiple of the alignment
    # strictly below the remainder, capped by max_context_chunk, fitting 'available'
    f = O.aligned_split_len
    assert f(0, 512, 256, 1024, 64) == 256        # printed example: request 1's head
    assert f(0, 512, 255, 1024, 64) == 192
    assert f(0, 512, 1000, 1024, 64) == 448        # below the remainder 512
    assert f(0, 30, 1024, 1024, 64) == 0           # nothing aligned below 30
    assert f(0, 65, 1024, 1024, 64) == 64
    assert f(0, 64, 1024, 1024, 64) == 0           # 64 itself is not a split of 64
    assert f(0, 131072, 65536, 65536, 64) == 65536
    assert f(0, 131072, 65536, 1000, 64) == 960    # capped by max_context_chunk
    assert f(128, 1000, 0, 1024, 64) == 0


def test_aligned_split_len_maximality():
    rng = np.random.default_rng(7)
    for _ in range(5000):
        a = int(rng.integers(1, 20))
        rem = int(rng.integers(1, 400))
        avail = int(rng.integers(0, 400))
        m = int(rng.integers(a, 400))
        s = O.aligned_split_len(int(rng.integers(0, 100)), rem, avail, m, a)
        assert s % a == 0 and 0 <= s < rem and s <= avail and s <= m
        nxt = s + a
        assert nxt >= rem or nxt > avail or nxt > m


def test_no_split_fits_closes_chunk():
    # reading: the chunk closes even when no aligned piece fits, so the
    # 1030 rows below never share one 1024-row chunk
    plans = _plan([1000, 30], 1024, 64)
    assert [(p.starts, p.seq_lens) for p in plans] == [([0], [1000]), ([0], [30])]


def test_zero_context_request_closes_chunk():
    # 131 rows would fit in 256, but request 32 has no context and chunks are
    # contiguous request slices
    wl = W.named_workloads()[2]
    plans = _plan(wl.context_lens, wl.workspace_rows, wl.split_alignment)
    assert [(p.request_start, p.request_end, sum(p.seq_lens)) for p in plans] == [(0, 32, 128), (33, 34, 3)]


def test_derived_plans():
    wls = W.named_workloads()
    p3 = _plan(wls[3].context_lens, 65536, 64)
    assert len(p3) == 1 and sum(p3[0].seq_lens) == 65536
    p5 = _plan(wls[5].context_lens, 65536, 64)
    assert len(p5) == 8
    assert [p.is_continuation for p in p5] == [False, True] * 4
    assert all(sum(p.seq_lens) == 65536 for p in p5)
    assert [(p.request_start, p.starts[0]) for p in p5] == [(r, s) for r in range(4) for s in (0, 65536)]


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        _plan([10], 8, 16)            # alignment above the budget
    with pytest.raises(ValueError):
        _plan([10], 16, 0)            # alignment below 1
    with pytest.raises(ValueError):
        _plan([10], 64, 16, 8)        # split cap below the alignment
    with pytest.raises(ValueError):
        _plan([-1], 64, 16)


def test_metadata_fields():
    wl = W.named_workloads()[1]
    md = O.build_chunked_context(wl.context_lens, wl.query_lens, wl.workspace_rows, wl.split_alignment)
    c0, c1 = md.chunks
    assert c0.cu_seq_lens.tolist() == [0, 768, 1024] and c1.cu_seq_lens.tolist() == [0, 256, 768]
    assert c0.max_seq_len == 768 and c1.max_seq_len == 512
    assert c0.max_query_len == 5 and c1.max_query_len == 7
    assert c0.token_to_seq.tolist() == [0] * 768 + [1] * 256
    assert c1.token_to_seq.tolist() == [0] * 256 + [1] * 512
    assert md.empty_token_slices == [(15, 19)]
    assert md.prefix_num_tokens == 15
    wl2 = W.named_workloads()[2]
    md2 = O.build_chunked_context(wl2.context_lens, wl2.query_lens, wl2.workspace_rows, wl2.split_alignment)
    assert md2.empty_token_slices == [(33, 164)]
    assert md2.prefix_num_tokens == 165
    assert [c.token_slice for c in md2.chunks] == [(0, 33), (164, 165)]
    assert O.build_chunked_context([0, 0], [3, 4], 64) is None
