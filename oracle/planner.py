"""Oracle: packing of context rows into workspace-sized chunks (integer, exact).

Follows the PR #50613 digest: section 实现拆解 (implementation breakdown)
items 1-2, and the plan_mla_context_chunks / aligned_split_len / _ContextChunkPlan
description in section 关键源码片段 (key source snippets).  The digest's listing
is taken as a description of what is computed; this is our own code.

Readings where the digest is silent or garbled (each also listed in the
design notes):
  * When the request at the front does not fit and an aligned split is taken,
    the chunk is closed.  When no aligned split fits, the chunk is closed as
    well (the listing's ``break`` sits inside the ``split_len > 0`` branch; read
    literally a whole request would then be appended past the budget, which
    contradicts the stated invariant that no chunk exceeds the workspace).
  * ``round_down(x, a)`` is floor(x / a) * a.
  * ``padded_rows`` defaults to the identity (workspace rows == context rows).
  * ``max_context_chunk`` defaults to the row budget; it caps split lengths only.
  * A request without context is never placed in a chunk, and it ends the
    chunk being filled, since a chunk covers a contiguous slice of requests.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional, Tuple

import numpy as np


def _identity(x: int) -> int:
    return x


def _round_down(x: int, a: int) -> int:
    return (x // a) * a


def aligned_split_len(start: int, remaining: int, available: int, max_context_chunk: int,
                      split_alignment: int, padded_rows: Callable[[int], int] = _identity) -> int:
    """Longest aligned head of a request's remaining context that fits.

    The candidate lengths are the multiples of ``split_alignment`` up to
    min(max_context_chunk, round_down(remaining - 1, split_alignment)) -- strictly
    shorter than ``remaining``, since a piece of full length is not a split.
    The answer is the largest candidate whose workspace rows
    padded_rows(start + L) - padded_rows(start) are <= ``available``, or 0.
    The digest finds it by binary search (valid because padded_rows is
    monotone); here every candidate is checked, which is the definition.
    """
    a = split_alignment
    limit = min(max_context_chunk, _round_down(remaining - 1, a))
    best = 0
    for m in range(0, limit // a + 1):
        length = m * a
        if padded_rows(start + length) - padded_rows(start) <= available:
            best = length
    return best


@dataclass
class ChunkPlan:
    """Layout of one chunk over request space (the digest's _ContextChunkPlan).

    ``starts[i]`` / ``seq_lens[i]`` are the context offset and row count of
    request ``request_start + i`` inside this chunk."""

    request_start: int
    request_end: int
    starts: List[int]
    seq_lens: List[int]
    is_continuation: bool


def plan_mla_context_chunks(context_lens, row_budget: int, max_context_chunk: Optional[int] = None,
                            split_alignment: int = 64,
                            padded_rows: Callable[[int], int] = _identity) -> List[ChunkPlan]:
    """Greedy, order-preserving packing of context rows into chunks.

    Requests are visited in order.  Each request with context contributes its
    remaining rows to the open chunk if they fit; otherwise its longest aligned
    head that fits (``aligned_split_len``) is placed and the chunk closes; the
    rest of that request opens the next chunk, which is then a continuation
    (its first entry starts at a nonzero offset).  Requests with no context are
    skipped and close the open chunk.
    """
    if max_context_chunk is None:
        max_context_chunk = row_budget
    if split_alignment < 1 or row_budget < split_alignment or max_context_chunk < split_alignment:
        raise ValueError("need 1 <= split_alignment <= row_budget and max_context_chunk >= split_alignment")
    lens = [int(c) for c in context_lens]
    if any(c < 0 for c in lens):
        raise ValueError("negative context length")

    plans: List[ChunkPlan] = []
    open_chunk = None  # [request_start, starts, seq_lens, rows]

    def close():
        nonlocal open_chunk
        if open_chunk is not None:
            rs, starts, seq_lens, _ = open_chunk
            assert seq_lens, "a chunk was closed before anything was placed in it"
            plans.append(ChunkPlan(rs, rs + len(seq_lens), starts, seq_lens, starts[0] > 0))
            open_chunk = None

    for req, ctx in enumerate(lens):
        if ctx == 0:
            close()
            continue
        pos = 0  # next context row of this request still to place
        while pos < ctx:
            if open_chunk is None:
                open_chunk = [req, [], [], 0]
            rest = ctx - pos
            rows_needed = padded_rows(ctx) - padded_rows(pos)
            room = row_budget - open_chunk[3]
            if rows_needed <= room:
                open_chunk[1].append(pos)
                open_chunk[2].append(rest)
                open_chunk[3] += rows_needed
                pos = ctx
            else:
                piece = aligned_split_len(pos, rest, room, max_context_chunk, split_alignment, padded_rows)
                if piece > 0:
                    open_chunk[1].append(pos)
                    open_chunk[2].append(piece)
                    open_chunk[3] += padded_rows(pos + piece) - padded_rows(pos)
                    pos += piece
                close()
    close()
    return plans


@dataclass
class ContextChunk:
    """Per-chunk metadata (the digest's ContextChunk, 实现拆解 items 1-4).

    request_slice / token_slice are half-open [begin, end) ranges over the
    batch's requests and prefill tokens.  cu_seq_lens[i] is the first workspace
    row of entry i (length n+1); token_to_seq[w] is the chunk-local entry that
    owns workspace row w; max_query_len is the longest query among the chunk's
    requests."""

    request_slice: Tuple[int, int]
    token_slice: Tuple[int, int]
    starts: np.ndarray
    seq_lens: np.ndarray
    cu_seq_lens: np.ndarray
    max_seq_len: int
    max_query_len: int
    token_to_seq: np.ndarray
    is_continuation: bool

    @property
    def num_rows(self) -> int:
        return int(self.cu_seq_lens[-1])


@dataclass
class ChunkedContextMetadata:
    """Flat chunk list plus the batch-wide fields (digest 实现拆解 item 1)."""

    chunks: List[ContextChunk]
    context_lens: np.ndarray
    query_start_loc: np.ndarray
    empty_token_slices: List[Tuple[int, int]] = field(default_factory=list)
    prefix_num_tokens: int = 0


def build_mla_chunked_context_metadata(plans: List[ChunkPlan], context_lens, query_lens) -> ChunkedContextMetadata:
    """Turn chunk plans into per-chunk tensors and the batch-wide fields.

    prefill_tokens_with_context (the merge threshold of the PR #36540 digest)
    is read as: the number of leading prefill tokens up to and including the
    last request that has context; every token past it has no context.
    empty_token_slices lists the token range of every request with no context.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    qsl = np.zeros(len(ql) + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(ql)
    chunks = []
    for p in plans:
        seq = np.asarray(p.seq_lens, dtype=np.int64)
        cu = np.zeros(len(seq) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(seq)
        owner = np.repeat(np.arange(len(seq), dtype=np.int64), seq)
        chunks.append(ContextChunk(
            request_slice=(p.request_start, p.request_end),
            token_slice=(int(qsl[p.request_start]), int(qsl[p.request_end])),
            starts=np.asarray(p.starts, dtype=np.int64),
            seq_lens=seq,
            cu_seq_lens=cu,
            max_seq_len=int(seq.max()),
            max_query_len=int(ql[p.request_start:p.request_end].max()) if p.request_end > p.request_start else 0,
            token_to_seq=owner,
            is_continuation=bool(p.is_continuation),
        ))
    empty = [(int(qsl[r]), int(qsl[r + 1])) for r in range(len(ctx)) if ctx[r] == 0]
    with_ctx = np.nonzero(ctx > 0)[0]
    prefix_num_tokens = int(qsl[with_ctx[-1] + 1]) if len(with_ctx) else 0
    return ChunkedContextMetadata(chunks, ctx, qsl, empty, prefix_num_tokens)


def build_chunked_context(context_lens, query_lens, workspace_rows: int, split_alignment: int = 64,
                          max_context_chunk: Optional[int] = None) -> Optional[ChunkedContextMetadata]:
    """Test helper of the same name on the PR #50613 digest: plan + metadata.

    Returns None when no request has context.  The digest's helper takes no
    split alignment; 64 (the paged block size of the workloads here) is used
    by default, and the printed example holds for any alignment dividing 256."""
    if not any(int(c) > 0 for c in context_lens):
        return None
    plans = plan_mla_context_chunks(context_lens, workspace_rows, max_context_chunk, split_alignment)
    return build_mla_chunked_context_metadata(plans, context_lens, query_lens)
