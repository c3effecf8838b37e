"""Pins of the oracle's gather, attention and merge against closed forms,
library routines and invariants (nothing here re-types the oracle's formulas).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as O
import workloads as W


# ---------------------------------------------------------------- gather


def test_gather_tagged_cache():
    """Each cache element holds a tag naming its (block, slot, head, dim); a
    gathered row must carry the tag of the physical place its logical position
    maps to, for every entry, across block boundaries and odd starts."""
    nb, bs, h, d = 23, 4, 2, 3
    tag = (np.arange(nb)[:, None, None, None] * 1_000_000 + np.arange(bs)[None, :, None, None] * 1000
           + np.arange(h)[None, None, :, None] * 10 + np.arange(d)[None, None, None, :])
    table = np.array([[5, 9, 2, 7, 11], [0, 22, 13, 4, 1], [3, 8, 6, 10, 12]], dtype=np.int32)
    reqs, starts, lens = [0, 1, 2], [8, 0, 3], [9, 4, 14]
    ws = O.gather_context_rows(tag, table, bs, reqs, starts, lens)
    assert ws.shape == (27, h, d)
    w = 0
    for r, s, n in zip(reqs, starts, lens):
        for j in range(n):
            pos = s + j
            blk, slot = table[r][pos // bs], pos % bs
            assert (ws[w] // 1000 == blk * 1000 + slot).all()
            assert ((ws[w] % 1000) == (np.arange(h)[:, None] * 10 + np.arange(d)[None, :])).all()
            w += 1


def test_gather_is_bit_copy():
    wl = W.named_workloads()[1]
    b = W.make_batch(wl)
    bits = b.k_cache.view(torch.int16).numpy()
    ws = O.gather_context_rows(bits, b.block_table.numpy(), wl.block_size, [0, 1], [0, 0], [768, 256])
    assert ws.dtype == np.int16
    table = b.block_table.numpy()
    assert (ws[0] == bits[table[0][0], 0]).all()
    assert (ws[767] == bits[table[0][767 // 64], 767 % 64]).all()
    assert (ws[768 + 255] == bits[table[1][255 // 64], 255 % 64]).all()


def test_gather_row_sources_by_hand():
    """Positions 2..8 of a request whose blocks are 5, 9, 2 (4 rows each):
    slots 2, 3 of block 5, then 0..3 of block 9, then 0 of block 2."""
    table = np.array([[5, 9, 2]], dtype=np.int32)
    src = O.gather_row_sources(table, 4, [0], [2], [7])
    assert src.tolist() == [22, 23, 36, 37, 38, 39, 8]
    assert O.gather_row_sources(table, 4, [], [], []).size == 0


def test_gather_row_sources_are_the_copied_rows():
    """The index map names exactly the rows the gather copies (tagged cache,
    several entries, odd starts, block boundaries)."""
    rng = np.random.default_rng(5)
    for bs in (1, 4, 16):
        nb, h, d = 40, 2, 3
        tag = np.arange(nb * bs * h * d, dtype=np.int64).reshape(nb, bs, h, d)
        table = np.stack([rng.permutation(nb)[:8] for _ in range(3)]).astype(np.int32)
        reqs = [2, 0, 1]
        starts = [int(rng.integers(0, 2 * bs)) for _ in reqs]
        lens = [int(rng.integers(1, 8 * bs - s + 1)) for s in starts]
        src = O.gather_row_sources(table, bs, reqs, starts, lens)
        ws = O.gather_context_rows(tag, table, bs, reqs, starts, lens)
        assert np.array_equal(tag.reshape(nb * bs, h, d)[src], ws)


# ------------------------------------------------------------- attention


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_key_closed_form():
    q, k, v = _rand((5, 3, 192), 1), _rand((1, 3, 192), 2), _rand((1, 3, 128), 3)
    scale = 1 / math.sqrt(192)
    out, lse = O.attention_with_lse(q, k, v, scale)
    assert np.allclose(out, np.broadcast_to(v, out.shape), rtol=0, atol=1e-14)
    s = scale * np.einsum("qhd,hd->hq", q, k[0])
    assert np.allclose(lse, s, rtol=0, atol=1e-12)


def test_equal_keys_closed_form():
    n = 37
    q, v = _rand((4, 2, 192), 4), _rand((n, 2, 128), 5)
    k = np.broadcast_to(_rand((1, 2, 192), 6), (n, 2, 192)).copy()
    out, lse = O.attention_with_lse(q, k, v, 0.1)
    assert np.allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)
    s = 0.1 * np.einsum("qhd,hd->hq", q, k[0])
    assert np.allclose(lse, math.log(n) + s, atol=1e-12)


def test_zero_query_closed_form():
    n = 19
    q, k, v = np.zeros((3, 1, 192)), _rand((n, 1, 192), 7), _rand((n, 1, 128), 8)
    out, lse = O.attention_with_lse(q, k, v, 0.3)
    assert np.allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)
    assert np.allclose(lse, math.log(n), atol=1e-13)


def test_no_keys_is_empty_state():
    out, lse = O.attention_with_lse(_rand((3, 2, 192), 1), np.zeros((0, 2, 192)), np.zeros((0, 2, 128)), 0.1)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_matches_torch_sdpa_and_logsumexp():
    """Library cross-check: torch's SDPA (fp64, CPU) for the output, scipy's
    logsumexp over torch-computed scores for the LSE."""
    nq, nk, h = 9, 41, 3
    q, k, v = _rand((nq, h, 192), 11), _rand((nk, h, 192), 12), _rand((nk, h, 128), 13)
    scale = 1 / math.sqrt(192)
    out, lse = O.attention_with_lse(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, atol=1e-12)
    scores = (torch.matmul(tq, tk.transpose(1, 2).contiguous()) * scale).numpy()
    assert np.allclose(lse, logsumexp(scores, axis=2), atol=1e-12)
    # causal against SDPA's causal mask (query i sees keys 0..i)
    k2, v2 = _rand((nq, h, 192), 14), _rand((nq, h, 128), 15)
    out_c, lse_c = O.attention_with_lse(q, k2, v2, scale, causal=True)
    tk2, tv2 = (torch.from_numpy(x).permute(1, 0, 2).contiguous() for x in (k2, v2))
    ref_c = torch.nn.functional.scaled_dot_product_attention(tq, tk2, tv2, scale=scale, is_causal=True)
    assert np.allclose(out_c, ref_c.permute(1, 0, 2).numpy(), atol=1e-12)
    sc = (torch.matmul(tq, tk2.transpose(1, 2).contiguous()) * scale).numpy()
    sc = np.where(np.tril(np.ones((nq, nq), dtype=bool))[None], sc, -np.inf)
    assert np.allclose(lse_c, logsumexp(sc, axis=2), atol=1e-12)


def test_causal_blocking_does_not_change_rows():
    q, k, v = _rand((23, 2, 192), 21), _rand((23, 2, 192), 22), _rand((23, 2, 128), 23)
    a = O.attention_with_lse(q, k, v, 0.07, causal=True)
    b = O.attention_with_lse(q, k, v, 0.07, causal=True, query_block=5)
    # BLAS may sum in a different order for a different matrix shape
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-13) and np.allclose(a[1], b[1], rtol=0, atol=1e-13)


# ----------------------------------------------------------------- merge


def _split_merge(q, k, v, cut, scale=0.1):
    a = O.attention_with_lse(q, k[:cut], v[:cut], scale)
    b = O.attention_with_lse(q, k[cut:], v[cut:], scale)
    return O.merge_states(a[0], a[1], b[0], b[1]), O.attention_with_lse(q, k, v, scale)


@pytest.mark.parametrize("cut", [1, 7, 20, 39])
def test_merge_of_disjoint_key_sets_is_union(cut):
    q, k, v = _rand((6, 3, 192), 31), _rand((40, 3, 192), 32), _rand((40, 3, 128), 33)
    (mo, ml), (fo, fl) = _split_merge(q, k, v, cut)
    assert np.allclose(mo, fo, atol=1e-13) and np.allclose(ml, fl, atol=1e-13)


def test_merge_with_empty_side_is_exact_and_never_reads_it():
    x_out, x_lse = _rand((5, 2, 8), 41), _rand((2, 5), 42)
    nan_out = np.full((5, 2, 8), np.nan)
    e_lse = np.full((2, 5), -np.inf)
    o, l = O.merge_states(x_out, x_lse, nan_out, e_lse)
    assert np.array_equal(o, x_out) and np.array_equal(l, x_lse)
    o, l = O.merge_states(nan_out, e_lse, x_out, x_lse)
    assert np.array_equal(o, x_out) and np.array_equal(l, x_lse)


def test_merge_both_empty_gives_zero_and_no_nan():
    # PR #49294 digest, 实现拆解 item 4: merging two empty states yields no NaN
    nan_out = np.full((4, 3, 16), np.nan)
    e = np.full((3, 4), -np.inf)
    o, l = O.merge_states(nan_out, e, nan_out.copy(), e)
    assert (o == 0).all() and np.isneginf(l).all()


def test_merge_commutative_and_associative():
    outs = [_rand((7, 2, 16), 50 + i) for i in range(3)]
    lses = [_rand((2, 7), 60 + i) * 3 for i in range(3)]
    lses[1][0, 2] = -np.inf
    ab = O.merge_states(outs[0], lses[0], outs[1], lses[1])
    ba = O.merge_states(outs[1], lses[1], outs[0], lses[0])
    assert np.allclose(ab[0], ba[0], atol=1e-15) and np.allclose(ab[1], ba[1], atol=1e-15)
    ab_c = O.merge_states(ab[0], ab[1], outs[2], lses[2])
    bc = O.merge_states(outs[1], lses[1], outs[2], lses[2])
    a_bc = O.merge_states(outs[0], lses[0], bc[0], bc[1])
    assert np.allclose(ab_c[0], a_bc[0], atol=1e-14) and np.allclose(ab_c[1], a_bc[1], atol=1e-14)


def test_merge_lse_closed_form():
    # equal LSEs: weights 1/2 each, LSE + ln 2
    a, b = _rand((3, 1, 4), 70), _rand((3, 1, 4), 71)
    l = np.full((1, 3), 1.25)
    o, lo = O.merge_states(a, l, b, l)
    assert np.allclose(o, (a + b) / 2, atol=1e-15) and np.allclose(lo, 1.25 + math.log(2), atol=1e-15)


def test_threshold_rows_copy_suffix_bit_exact():
    # PR #36540 digest, 实现拆解: rows at or past prefix_num_tokens take the suffix
    p_out, p_lse = _rand((10, 2, 8), 80), _rand((2, 10), 81)
    s_out, s_lse = _rand((10, 2, 8), 82), _rand((2, 10), 83)
    p_out[6:] = np.nan  # rows past the threshold are never read on the prefix side
    o, l = O.merge_attn_states(p_out, p_lse, s_out, s_lse, prefix_num_tokens=6)
    assert np.array_equal(o[6:], s_out[6:]) and np.array_equal(l[:, 6:], s_lse[:, 6:])
    ref = O.merge_states(p_out[:6], p_lse[:, :6], s_out[:6], s_lse[:, :6])
    assert np.array_equal(o[:6], ref[0]) and np.array_equal(l[:, :6], ref[1])


def test_init_partial():
    o, l = O.init_mla_context_partial(3, 2, 5)
    assert o.shape == (3, 2, 5) and (o == 0).all() and l.shape == (2, 3) and np.isneginf(l).all()
