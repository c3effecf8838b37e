"""Oracle: chunk planning and context gathering under decode context
parallelism (DCP), emulated on one device.  TEST INFRASTRUCTURE ONLY (see the
package docstring).

The PR #50613 digest names the parts (实现拆解 item 5: the test file covers
"DCP local chunks"; 风险与影响: local chunk planning with padded_local_* and
local_starts, and all ranks must agree or the all-gather misaligns) and the
planner's padded_rows hook (关键源码片段); it prints neither the sharding nor
padded_rows.  Readings (each also in the design notes):

  * D ranks hold each request's context interleaved in runs of I positions:
    position p is on rank (p // I) % D, at local index
    (p // (I * D)) * I + p % I of that rank's own paged cache.
  * Every rank pads its local rows of a context prefix x to the most any rank
    holds, padded_local(x) = I * ceil(x / (I * D)), so all ranks build the
    same plan and contribute equal-sized workspaces to the all-gather.
  * The planner counts rows of the all-gathered workspace:
    padded_rows(x) = D * padded_local(x).
  * The split alignment is a multiple of I * D, so every entry starts at the
    start of a round of rank runs and its local start on every rank is
    start / D.
  * Per chunk, rank r gathers local rows [start_i / D, padded_local(start_i +
    len_i)) of each entry i into its workspace at cu_local[i]; the all-gather
    stacks the D workspaces (L = cu_local[-1] rows each); the reorganisation
    reads position p of entry i from row r * L + cu_local[i] + local(p) -
    start_i / D and writes the chunk's rows in request order, which is what
    the single-device gather produces.  Local rows past what a rank holds
    are padding and never read.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention_with_lse, gather_context_rows
from .merge import accumulate_mla_context_chunk, init_mla_context_partial, merge_attn_states
from .planner import plan_mla_context_chunks


def dcp_owner(p: int, world: int, interleave: int) -> int:
    return (p // interleave) % world


def dcp_local_index(p: int, world: int, interleave: int) -> int:
    return (p // (interleave * world)) * interleave + p % interleave


def padded_local_rows(x: int, world: int, interleave: int) -> int:
    """Local rows every rank reserves for context positions [0, x)."""
    return interleave * math.ceil(x / (interleave * world))


def plan_dcp_context_chunks(context_lens, row_budget: int, split_alignment: int, world: int,
                            interleave: int = 1, max_context_chunk=None):
    """plan_mla_context_chunks with padded_rows(x) = D * padded_local(x)."""
    if world < 1 or interleave < 1 or split_alignment % (world * interleave) != 0:
        raise ValueError("split_alignment must be a multiple of world * interleave")
    return plan_mla_context_chunks(context_lens, row_budget, max_context_chunk, split_alignment,
                                   lambda x: world * padded_local_rows(x, world, interleave))


def dcp_local_entries(plan, world: int, interleave: int):
    """local_starts, padded local lengths and their offsets cu_local of one chunk."""
    starts = [s // world for s in plan.starts]
    lens = [padded_local_rows(s + n, world, interleave) - s // world for s, n in zip(plan.starts, plan.seq_lens)]
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    return starts, lens, cu


def local_context_lens(context_lens, rank: int, world: int, interleave: int):
    """Context positions each request has on one rank."""
    return [sum(1 for p in range(int(c)) if dcp_owner(p, world, interleave) == rank) for c in context_lens]


def gather_local_rows(cache, block_table, block_size, request_ids, local_starts, local_lens, held):
    """One rank's gather of a chunk: the padded local rows of each entry, with
    rows past what the rank holds (``held`` per request) left NaN."""
    pieces = []
    for r, s, n in zip(request_ids, local_starts, local_lens):
        real = max(0, min(n, int(held[r]) - s))
        rows = gather_context_rows(cache, block_table, block_size, [r], [s], [real]).astype(np.float64)
        pad = np.full((n - real,) + cache.shape[2:], np.nan)
        pieces.append(np.concatenate([rows, pad], axis=0))
    return np.concatenate(pieces, axis=0) if pieces else np.zeros((0,) + cache.shape[2:])


def reorganize(gathered, plan, cu_local, world: int, interleave: int):
    """Rows of the all-gathered workspace [world * L, ...] back in request
    order: entry i's position p comes from its owner's block."""
    L = int(cu_local[-1])
    out = []
    for i, (s, n) in enumerate(zip(plan.starts, plan.seq_lens)):
        for p in range(s, s + n):
            r = dcp_owner(p, world, interleave)
            out.append(gathered[r * L + int(cu_local[i]) + dcp_local_index(p, world, interleave) - s // world])
    return np.stack(out) if out else gathered[:0]


def dcp_chunked_prefill(q, k_new, v_new, local_k, local_v, local_tables, block_size, context_lens, query_lens,
                        workspace_rows, split_alignment, scale, world, interleave=1):
    """The chunked path with every chunk's rows assembled as under DCP.

    local_k[r] / local_v[r] / local_tables[r]: rank r's paged caches and block
    table (request r's local positions in order).  Returns the same dict as
    ``chunked_prefill`` plus the plans."""
    ctx = [int(c) for c in context_lens]
    ql = [int(x) for x in query_lens]
    T, H, dv = q.shape[0], q.shape[1], v_new.shape[2]
    qsl = np.zeros(len(ql) + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(ql)
    plans = plan_dcp_context_chunks(ctx, workspace_rows, split_alignment, world, interleave)
    held = [local_context_lens(ctx, r, world, interleave) for r in range(world)]
    p_out, p_lse = init_mla_context_partial(T, H, dv)
    for pl in plans:
        req_ids = list(range(pl.request_start, pl.request_end))
        ls, ln, cu_local = dcp_local_entries(pl, world, interleave)
        assert world * int(cu_local[-1]) <= workspace_rows, "chunk exceeds the workspace"
        gk = np.concatenate([gather_local_rows(local_k[r], local_tables[r], block_size, req_ids, ls, ln, held[r])
                             for r in range(world)])
        gv = np.concatenate([gather_local_rows(local_v[r], local_tables[r], block_size, req_ids, ls, ln, held[r])
                             for r in range(world)])
        ws_k = reorganize(gk, pl, cu_local, world, interleave)
        ws_v = reorganize(gv, pl, cu_local, world, interleave)
        t0, t1 = int(qsl[pl.request_start]), int(qsl[pl.request_end])
        c_out = np.zeros((t1 - t0, H, dv))
        c_lse = np.full((H, t1 - t0), -np.inf)
        k0 = 0
        for i, r in enumerate(req_ids):
            a, b = int(qsl[r]) - t0, int(qsl[r + 1]) - t0
            n = pl.seq_lens[i]
            o, l = attention_with_lse(q[t0 + a:t0 + b], ws_k[k0:k0 + n], ws_v[k0:k0 + n], scale)
            c_out[a:b] = o
            c_lse[:, a:b] = l
            k0 += n
        accumulate_mla_context_chunk(p_out, p_lse, c_out, c_lse, (t0, t1))
    s_out = np.zeros((T, H, dv))
    s_lse = np.full((H, T), -np.inf)
    for r in range(len(ql)):
        a, b = int(qsl[r]), int(qsl[r + 1])
        o, l = attention_with_lse(q[a:b], k_new[a:b], v_new[a:b], scale, causal=True)
        s_out[a:b] = o
        s_lse[:, a:b] = l
    with_ctx = [r for r in range(len(ctx)) if ctx[r] > 0]
    prefix = int(qsl[with_ctx[-1] + 1]) if with_ctx else 0
    out, lse = merge_attn_states(p_out, p_lse, s_out, s_lse, prefix)
    return dict(out=out, lse=lse, partial_out=p_out, partial_lse=p_lse, plans=plans)
