"""Oracle: the uniform-window context scheduler, i.e. the scheduling that
per-request chunk packing replaced (PR #50613 digest, 功能与动机), with the
empty-context mask of the PR #49294 digest in its loop.  TEST INFRASTRUCTURE
ONLY (see the package docstring).

Scheduler (PR #50613 digest, 功能与动机): the workspace of W rows is shared
equally by the requests that have context.  Each gets a window of
    w = floor(floor(W / n_ctx) / A) * A
rows (reading: A is the paged block size so windows start on block
boundaries; A = 1 leaves the plain equal share), and iteration i covers
context rows [i*w, (i+1)*w) of every request.  The loop runs
ceil(max_ctx / w) times and every iteration attends and merges over the whole
prefill batch, also for requests whose window is already empty.

One iteration (PR #49294 digest, 实现拆解 items 2-3):
  gather every request's window rows into the workspace;
  attention of each request's queries against its window rows; a request
  whose window is empty gets an unspecified result from the attention
  backend, NaN here (as in the digest's test);
  if any window of the iteration is empty, mask_empty_context over the
  iteration's result with this iteration's cu_seq_lens;
  iteration 0's result becomes the context state, every later result is
  LSE-merged into it over all tokens.
The causal suffix and the thresholded final merge are those of the chunked
path.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention_with_lse, gather_context_rows
from .mask import mask_empty_context
from .merge import merge_attn_states, merge_states


def uniform_window_size(context_lens, workspace_rows: int, split_alignment: int = 1) -> int:
    """Window rows per request; 0 when no request has context.

    Raises ValueError when the equal share is smaller than one aligned window
    (the earlier scheduler needed a workspace of at least one block per
    request with context, PR #50613 digest, 实现拆解 item 5)."""
    if split_alignment < 1 or workspace_rows < 1:
        raise ValueError("workspace_rows and split_alignment must be >= 1")
    n_ctx = sum(1 for c in context_lens if int(c) > 0)
    if n_ctx == 0:
        return 0
    share = workspace_rows // n_ctx
    w = (share // split_alignment) * split_alignment
    if w < 1:
        raise ValueError(f"workspace of {workspace_rows} rows gives no aligned window for {n_ctx} requests")
    return w


def plan_uniform_windows(context_lens, workspace_rows: int, split_alignment: int = 1):
    """Returns (w, starts, seq_lens): starts and seq_lens are [iterations][N]
    lists; seq_lens[i][r] = max(0, min(ctx_r, (i+1)w) - i*w) and
    starts[i][r] = i*w."""
    ctx = [int(c) for c in context_lens]
    w = uniform_window_size(ctx, workspace_rows, split_alignment)
    if w == 0:
        return 0, [], []
    iters = math.ceil(max(ctx) / w)
    starts = [[i * w] * len(ctx) for i in range(iters)]
    seq_lens = [[max(0, min(c, (i + 1) * w) - i * w) for c in ctx] for i in range(iters)]
    return w, starts, seq_lens


def uniform_window_prefill(q, k_new, v_new, k_cache, v_cache, block_table, block_size, context_lens,
                           query_lens, workspace_rows, split_alignment, scale, skip_mask=False):
    """Prefill with the uniform-window scheduler.  Same arrays and return
    dict as ``chunked_prefill`` (plus ``window`` and ``iterations``).
    ``skip_mask`` drops the mask step (a planted mistake for the tests)."""
    ctx = [int(c) for c in context_lens]
    ql = [int(x) for x in query_lens]
    N = len(ctx)
    T, H, dv = q.shape[0], q.shape[1], v_new.shape[2]
    qsl = np.zeros(N + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(ql)
    w, starts, seq_lens = plan_uniform_windows(ctx, workspace_rows, split_alignment)

    p_out = p_lse = None
    for it in range(len(seq_lens)):
        lens = seq_lens[it]
        cu = np.zeros(N + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lens)
        assert cu[-1] <= workspace_rows, "iteration exceeds the workspace"
        ws_k = gather_context_rows(k_cache, block_table, block_size, list(range(N)), starts[it], lens)
        ws_v = gather_context_rows(v_cache, block_table, block_size, list(range(N)), starts[it], lens)
        c_out = np.full((T, H, dv), np.nan, dtype=np.float64)
        c_lse = np.full((H, T), np.nan, dtype=np.float64)
        for r in range(N):
            a, b = int(qsl[r]), int(qsl[r + 1])
            if lens[r] == 0 or a == b:
                continue  # the backend's result for an empty window is unspecified
            o, l = attention_with_lse(q[a:b], ws_k[cu[r]:cu[r + 1]], ws_v[cu[r]:cu[r + 1]], scale)
            c_out[a:b] = o
            c_lse[:, a:b] = l
        if any(x == 0 for x in lens) and not skip_mask:
            mask_empty_context(c_lse, c_out, qsl, cu)
        if it == 0:
            p_out, p_lse = c_out, c_lse
        else:
            p_out, p_lse = merge_states(p_out, p_lse, c_out, c_lse)

    s_out = np.zeros((T, H, dv), dtype=np.float64)
    s_lse = np.full((H, T), -np.inf, dtype=np.float64)
    for r in range(N):
        a, b = int(qsl[r]), int(qsl[r + 1])
        o, l = attention_with_lse(q[a:b], k_new[a:b], v_new[a:b], scale, causal=True)
        s_out[a:b] = o
        s_lse[:, a:b] = l

    with_ctx = [r for r in range(N) if ctx[r] > 0]
    prefix_num_tokens = int(qsl[with_ctx[-1] + 1]) if with_ctx else 0
    if p_out is None:  # no context anywhere: the final merge reads no prefix row
        p_out = np.zeros((T, H, dv), dtype=np.float64)
        p_lse = np.full((H, T), -np.inf, dtype=np.float64)
    out, lse = merge_attn_states(p_out, p_lse, s_out, s_lse, prefix_num_tokens)
    return dict(out=out, lse=lse, partial_out=p_out, partial_lse=p_lse, suffix_out=s_out, suffix_lse=s_lse,
                window=w, iterations=len(seq_lens), prefix_num_tokens=prefix_num_tokens)
