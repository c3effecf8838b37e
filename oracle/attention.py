"""Oracle: paged-cache gather and naive softmax attention with LSE (fp64).

Gather: every context row of every chunk entry is copied once from the paged
cache into consecutive workspace rows (PR #50613 digest, 实现拆解 item 2: each
context row is gathered exactly once).  A context position p of request r
lives in physical block block_table[r][p // B] at slot p % B.

Attention: for query q and keys k_j, s_j = scale * (q . k_j), the output is
sum_j softmax(s)_j v_j and LSE = ln sum_j exp(s_j).  The digests do not print
a formula; this is the standard definition the backends compute, checked on
the PR #50613 digest (实现拆解 item 5) against an SDPA reference.  LSE is the
natural log of the scaled scores, one value per (head, token), stored
head-major [H, T] as in the merge tests of the PR #49294 digest.  A query
with no keys gets output 0 and LSE -inf.
"""
from __future__ import annotations

import numpy as np


def gather_context_rows(cache: np.ndarray, block_table: np.ndarray, block_size: int,
                        request_ids, starts, seq_lens) -> np.ndarray:
    """Copy the context rows of one chunk out of a paged cache.

    cache: [num_blocks, block_size, H, D]; entry i takes rows
    starts[i] .. starts[i]+seq_lens[i]-1 of request request_ids[i].
    Returns [sum(seq_lens), H, D] (a bit copy: same dtype as the cache)."""
    pieces = []
    for r, s, n in zip(request_ids, starts, seq_lens):
        pos = np.arange(int(s), int(s) + int(n), dtype=np.int64)
        blocks = np.asarray(block_table)[int(r)][pos // block_size].astype(np.int64)
        pieces.append(cache[blocks, pos % block_size])
    if not pieces:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.concatenate(pieces, axis=0)


def gather_row_sources(block_table: np.ndarray, block_size: int, request_ids, starts, seq_lens) -> np.ndarray:
    """Where each workspace row of one chunk comes from, as a flat cache row
    index (physical block * block_size + slot), in workspace order: entry i
    takes positions starts[i] .. starts[i]+seq_lens[i]-1 of request
    request_ids[i], and position p lives at slot p % B of physical block
    block_table[r][p // B].  gather_context_rows copies exactly these rows."""
    pieces = []
    for r, s, n in zip(request_ids, starts, seq_lens):
        pos = np.arange(int(s), int(s) + int(n), dtype=np.int64)
        blocks = np.asarray(block_table)[int(r)][pos // block_size].astype(np.int64)
        pieces.append(blocks * block_size + pos % block_size)
    if not pieces:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(pieces)


def _attend_one_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """q [nq, dk], k [nk, dk], v [nk, dv] -> out [nq, dv], lse [nq] (fp64)."""
    nq, nk = q.shape[0], k.shape[0]
    out = np.zeros((nq, v.shape[1]), dtype=np.float64)
    lse = np.full(nq, -np.inf, dtype=np.float64)
    if nq == 0 or nk == 0:
        return out, lse
    s = scale * (q @ k.T)  # [nq, nk]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ v) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def attention_with_lse(q, k, v, scale: float, causal: bool = False, query_block: int = 4096):
    """Attention of one sequence, all heads.

    q [nq, H, dk], k [nk, H, dk], v [nk, H, dv] (any float dtype; computed in
    float64) -> out [nq, H, dv] float64, lse [H, nq] float64.  Queries are
    processed ``query_block`` at a time only to bound memory; each query row is
    computed the same way regardless."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, H = q.shape[0], q.shape[1]
    out = np.zeros((nq, H, v.shape[2]), dtype=np.float64)
    lse = np.full((H, nq), -np.inf, dtype=np.float64)
    for h in range(H):
        kh, vh = k[:, h, :], v[:, h, :]
        for q0 in range(0, nq, query_block):
            q1 = min(nq, q0 + query_block)
            if causal:
                o, l = _attend_causal_block(q[q0:q1, h, :], kh, vh, scale, q0)
            else:
                o, l = _attend_one_head(q[q0:q1, h, :], kh, vh, scale)
            out[q0:q1, h, :] = o
            lse[h, q0:q1] = l
    return out, lse


def _attend_causal_block(q, k, v, scale, q0):
    """Causal rows q0.. of a sequence: query q0+i sees keys 0..q0+i."""
    nq = q.shape[0]
    nk = q0 + nq
    if nk == 0:
        return np.zeros((nq, v.shape[1])), np.full(nq, -np.inf)
    s = scale * (q @ k[:nk].T)
    visible = np.arange(nk)[None, :] <= (q0 + np.arange(nq))[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v[:nk]) / l, (m + np.log(l))[:, 0]
