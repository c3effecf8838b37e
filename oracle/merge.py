"""Oracle: merging attention partials by their log-sum-exp (fp64).

Two partial results (O_a, L_a) and (O_b, L_b) of attention over disjoint key
sets combine into the result over the union:
    L = ln(e^L_a + e^L_b),   O = (e^L_a O_a + e^L_b O_b) / e^L.
An empty side has L = -inf and contributes nothing; its output is never read
(it may be garbage or NaN: the PR #36540 digest leaves chunk outputs
uninitialised, and the PR #49294 digest's test fills empty rows with NaN).  Two
empty sides give (0, -inf) and never NaN (PR #49294 digest, 实现拆解 item 4).

merge_attn_states takes a threshold prefix_num_tokens: token rows at or past it
take the suffix verbatim (PR #36540 digest, 实现拆解, CUDA kernel layer).

Partials live in an output [T, H, D] and an LSE [H, T] (head-major).
"""
from __future__ import annotations

import numpy as np


def merge_states(a_out, a_lse, b_out, b_lse):
    """Elementwise LSE merge.  a_out/b_out [T, H, D], a_lse/b_lse [H, T].

    Returns (out [T, H, D] float64, lse [H, T] float64)."""
    a_out = np.asarray(a_out, dtype=np.float64)
    b_out = np.asarray(b_out, dtype=np.float64)
    a_lse = np.asarray(a_lse, dtype=np.float64)
    b_lse = np.asarray(b_lse, dtype=np.float64)
    a_empty = np.isneginf(a_lse).T[:, :, None]  # [T, H, 1]
    b_empty = np.isneginf(b_lse).T[:, :, None]
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.maximum(a_lse, b_lse)
        m_safe = np.where(np.isneginf(m), 0.0, m)
        wa = np.exp(a_lse - m_safe)  # 0 for an empty side
        wb = np.exp(b_lse - m_safe)
        tot = wa + wb
        lse = np.where(np.isneginf(m), -np.inf, m_safe + np.log(np.where(tot > 0, tot, 1.0)))
        fa = (wa / np.where(tot > 0, tot, 1.0)).T[:, :, None]
        fb = (wb / np.where(tot > 0, tot, 1.0)).T[:, :, None]
        both = fa * a_out + fb * b_out
    # select, never multiply an unread side by zero: NaN in it must not leak
    out = np.where(a_empty & b_empty, 0.0, np.where(a_empty, b_out, np.where(b_empty, a_out, both)))
    return out, lse


def merge_attn_states(prefix_out, prefix_lse, suffix_out, suffix_lse, prefix_num_tokens=None):
    """Final merge.  Rows t >= prefix_num_tokens copy the suffix row and LSE;
    earlier rows are merged with ``merge_states``."""
    out, lse = merge_states(prefix_out, prefix_lse, suffix_out, suffix_lse)
    T = out.shape[0]
    k = T if prefix_num_tokens is None else int(prefix_num_tokens)
    if k < T:
        out[k:] = np.asarray(suffix_out, dtype=np.float64)[k:]
        lse[:, k:] = np.asarray(suffix_lse, dtype=np.float64)[:, k:]
    return out, lse


def init_mla_context_partial(num_tokens: int, num_heads: int, head_dim: int):
    """Context partial for every prefill token: output 0, LSE -inf
    (PR #50613 digest, 实现拆解 item 3)."""
    return (np.zeros((num_tokens, num_heads, head_dim), dtype=np.float64),
            np.full((num_heads, num_tokens), -np.inf, dtype=np.float64))


def accumulate_mla_context_chunk(partial_out, partial_lse, chunk_out, chunk_lse, token_slice):
    """Merge one chunk's (output, LSE) into the partial rows of its token
    slice, in place (PR #50613 digest, 实现拆解 item 3)."""
    t0, t1 = token_slice
    o, l = merge_states(partial_out[t0:t1], partial_lse[:, t0:t1], chunk_out, chunk_lse)
    partial_out[t0:t1] = o
    partial_lse[:, t0:t1] = l
