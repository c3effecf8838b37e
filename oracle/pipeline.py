"""Oracle: chunked-context prefill end to end, and its direct definition.

Chunked path (PR #50613 digest, 实现拆解 items 2-3; PR #36540 digest for the
final merge):
  1. plan chunks and build their metadata on the host;
  2. init the context partial for all T prefill tokens to (0, -inf);
  3. per chunk: gather its context rows into a workspace, run non-causal
     attention of each request's queries against that request's rows, and
     LSE-merge the chunk result into the partial rows of the chunk's tokens;
  4. causal attention of each request's new tokens over its new tokens
     (the "suffix"; query i sees new tokens 0..i of its own request);
  5. merge_attn_states(partial, suffix, prefix_num_tokens).

Direct definition (no chunks, no merges): token i of request r with context
length c attends to context rows 0..c-1 and new tokens 0..i of r, in one
softmax.  Up to rounding the chunked path equals it; the tests pin that.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_with_lse, gather_context_rows
from .merge import accumulate_mla_context_chunk, init_mla_context_partial, merge_attn_states
from .planner import build_mla_chunked_context_metadata, plan_mla_context_chunks


def chunked_prefill(q, k_new, v_new, k_cache, v_cache, block_table, block_size, context_lens,
                    query_lens, workspace_rows, split_alignment, scale, max_context_chunk=None,
                    keep_workspaces=False):
    """Run the chunked path.  Arrays are token-major ([T, H, D]) and the caches
    paged ([NB, B, H, D]); values are used as float64.

    Returns a dict: out [T,H,dv], lse [H,T], partial_out/partial_lse (context
    partial), suffix_out/suffix_lse, metadata, and (optionally) the gathered
    workspaces of each chunk."""
    ctx = [int(c) for c in context_lens]
    ql = [int(x) for x in query_lens]
    T, H, dv = q.shape[0], q.shape[1], v_new.shape[2]
    plans = plan_mla_context_chunks(ctx, workspace_rows, max_context_chunk, split_alignment)
    md = build_mla_chunked_context_metadata(plans, ctx, ql)
    qsl = md.query_start_loc

    p_out, p_lse = init_mla_context_partial(T, H, dv)
    workspaces = []
    for ch in md.chunks:
        rs, re_ = ch.request_slice
        assert ch.num_rows <= workspace_rows, "chunk exceeds the workspace"
        req_ids = list(range(rs, re_))
        ws_k = gather_context_rows(k_cache, block_table, block_size, req_ids, ch.starts, ch.seq_lens)
        ws_v = gather_context_rows(v_cache, block_table, block_size, req_ids, ch.starts, ch.seq_lens)
        if keep_workspaces:
            workspaces.append((ws_k, ws_v))
        t0, t1 = ch.token_slice
        c_out = np.zeros((t1 - t0, H, dv), dtype=np.float64)
        c_lse = np.full((H, t1 - t0), -np.inf, dtype=np.float64)
        for i, r in enumerate(req_ids):
            a, b = int(qsl[r]) - t0, int(qsl[r + 1]) - t0
            k0, k1 = int(ch.cu_seq_lens[i]), int(ch.cu_seq_lens[i + 1])
            o, l = attention_with_lse(q[t0 + a:t0 + b], ws_k[k0:k1], ws_v[k0:k1], scale)
            c_out[a:b] = o
            c_lse[:, a:b] = l
        accumulate_mla_context_chunk(p_out, p_lse, c_out, c_lse, ch.token_slice)

    s_out = np.zeros((T, H, dv), dtype=np.float64)
    s_lse = np.full((H, T), -np.inf, dtype=np.float64)
    for r in range(len(ql)):
        a, b = int(qsl[r]), int(qsl[r + 1])
        o, l = attention_with_lse(q[a:b], k_new[a:b], v_new[a:b], scale, causal=True)
        s_out[a:b] = o
        s_lse[:, a:b] = l

    out, lse = merge_attn_states(p_out, p_lse, s_out, s_lse, md.prefix_num_tokens)
    return dict(out=out, lse=lse, partial_out=p_out, partial_lse=p_lse, suffix_out=s_out,
                suffix_lse=s_lse, metadata=md, workspaces=workspaces)


def _context_rows_of(cache, block_table, block_size, request, length):
    """Rows 0..length-1 of a request, read block by block from the cache."""
    rows = []
    for b in range((length + block_size - 1) // block_size):
        take = min(block_size, length - b * block_size)
        rows.append(np.asarray(cache[int(block_table[request][b])][:take], dtype=np.float64))
    if not rows:
        return np.zeros((0,) + tuple(cache.shape[2:]), dtype=np.float64)
    return np.concatenate(rows, axis=0)


def direct_prefill(q, k_new, v_new, k_cache, v_cache, block_table, block_size, context_lens,
                   query_lens, scale, requests=None, query_block=None):
    """The definition computed directly: one softmax per (token, head) over
    the request's context rows followed by its new tokens up to itself.

    Returns out [T, H, dv] and lse [H, T] (rows of requests not listed in
    ``requests`` are left 0 / -inf).  ``query_block`` only bounds memory: a
    request's tokens are taken that many at a time, each row computed the
    same way."""
    T, H, dv = q.shape[0], q.shape[1], v_new.shape[2]
    ql = [int(x) for x in query_lens]
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int64)
    out = np.zeros((T, H, dv), dtype=np.float64)
    lse = np.full((H, T), -np.inf, dtype=np.float64)
    for r in (range(len(ql)) if requests is None else requests):
        c = int(context_lens[r])
        a, b = int(qsl[r]), int(qsl[r + 1])
        n = b - a
        if n == 0:
            continue
        kc = _context_rows_of(k_cache, block_table, block_size, r, c)
        vc = _context_rows_of(v_cache, block_table, block_size, r, c)
        k_all = np.concatenate([kc, np.asarray(k_new[a:b], dtype=np.float64)], axis=0)
        v_all = np.concatenate([vc, np.asarray(v_new[a:b], dtype=np.float64)], axis=0)
        qr = np.asarray(q[a:b], dtype=np.float64)
        key_pos = np.arange(c + n)
        step = n if query_block is None else int(query_block)
        for t0 in range(0, n, step):
            t1 = min(n, t0 + step)
            visible = key_pos[None, :] < (c + 1 + np.arange(t0, t1))[:, None]  # [t1-t0, c+n]
            for h in range(H):
                s = scale * (qr[t0:t1, h, :] @ k_all[:, h, :].T)
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                out[a + t0:a + t1, h, :] = (e @ v_all[:, h, :]) / l
                lse[h, a + t0:a + t1] = (m + np.log(l))[:, 0]
    return out, lse


def direct_rows(q_rows, positions, k_ctx, v_ctx, k_new, v_new, scale):
    """The definition for selected tokens of one request.

    q_rows [n, H, dk]: the queries of the selected tokens; positions [n]: each
    token's index among the request's new tokens; k_ctx/v_ctx [c, H, d]: the
    request's context rows in order; k_new/v_new [>= max(positions)+1, H, d]:
    its new tokens.  Token i attends to all c context rows and new tokens
    0..positions[i].  Returns out [n, H, dv] and lse [H, n] (float64)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    n, H = q_rows.shape[0], q_rows.shape[1]
    c = k_ctx.shape[0]
    out = np.zeros((n, H, v_new.shape[2]), dtype=np.float64)
    lse = np.full((H, n), -np.inf, dtype=np.float64)
    k_all = np.concatenate([np.asarray(k_ctx, dtype=np.float64), np.asarray(k_new, dtype=np.float64)], axis=0)
    v_all = np.concatenate([np.asarray(v_ctx, dtype=np.float64), np.asarray(v_new, dtype=np.float64)], axis=0)
    for i, pos in enumerate(positions):
        visible = c + int(pos) + 1
        for h in range(H):
            s = scale * (k_all[:visible, h, :] @ q_rows[i, h, :])
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            out[i, h, :] = (e @ v_all[:visible, h, :]) / l
            lse[h, i] = m + np.log(l)
    return out, lse
