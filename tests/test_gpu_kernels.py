"""GPU parity of each kernel against the oracle, through the C ABI.

merge and gather: bit-exact where the result is a copy or a select, within
fp32-then-bf16 rounding where it is arithmetic.  Attention: the output/LSE
bars of gpu_util, on ragged varlen batches spanning several query and key
tiles, empty sequences and causal masks.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import OUT_TOL, check, host, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


# ------------------------------------------------------------------- merge


@pytest.mark.parametrize("head_dim", [128, 16, 72])
@pytest.mark.parametrize("threshold", [None, 0, 23])
def test_merge_matches_oracle(head_dim, threshold):
    say(f"merge head_dim={head_dim} threshold={threshold}")
    g = torch.Generator().manual_seed(7 + head_dim)
    T, H = 41, 5
    po = torch.randn(T, H, head_dim, generator=g).to(torch.bfloat16)
    so = torch.randn(T, H, head_dim, generator=g).to(torch.bfloat16)
    pl = (torch.randn(H, T, generator=g) * 3).float()
    sl = (torch.randn(H, T, generator=g) * 3).float()
    # empty states with NaN outputs: prefix only, suffix only, both
    pl[0, 3] = -float("inf"); po[3, 0] = float("nan")
    sl[1, 4] = -float("inf"); so[4, 1] = float("nan")
    pl[2, 5] = sl[2, 5] = -float("inf"); po[5, 2] = so[5, 2] = float("nan")
    pl[:, 30:] = -float("inf"); po[30:] = float("nan")
    ref_o, ref_l = O.merge_attn_states(host(po), pl.double().numpy(), host(so), sl.double().numpy(),
                                       threshold if threshold is not None else T)
    d = [x.to(DEV) for x in (po, pl, so, sl)]
    out = torch.full_like(d[0], float("nan"))
    out_l = torch.full_like(d[1], float("nan"))
    mla.mla_merge_attn_states(out, out_l, d[0], d[1], d[2], d[3], threshold)
    torch.cuda.synchronize()
    o, l = host(out), out_l.double().cpu().numpy()
    # NaN only where a row is copied verbatim from a NaN input (as in the oracle)
    assert np.array_equal(np.isnan(o), np.isnan(ref_o)) and not np.isnan(l).any()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(l[fin] - ref_l[fin]).max() < 1e-5
    # copies and selects are bit-exact
    ob, pb, sb = _bits(out), _bits(po), _bits(so)
    pl, sl = pl.numpy(), sl.numpy()
    k = T if threshold is None else threshold
    for t in range(T):
        for h in range(H):
            if t >= k or (np.isneginf(pl[h, t]) and not np.isneginf(sl[h, t])):
                assert (ob[t, h] == sb[t, h]).all(), (t, h)
            elif np.isneginf(sl[h, t]) and not np.isneginf(pl[h, t]):
                assert (ob[t, h] == pb[t, h]).all(), (t, h)
            elif np.isneginf(sl[h, t]) and np.isneginf(pl[h, t]):
                assert (o[t, h] == 0).all()
    # weighted rows: fp32 math then one bf16 rounding
    scale = np.maximum(np.abs(host(po)), np.abs(host(so)))
    scale = np.where(np.isnan(scale), 0, scale)
    ok = np.isnan(ref_o) | (np.abs(o - ref_o) <= 2.0 ** -7 * np.maximum(scale, np.abs(ref_o)) + 1e-6)
    assert ok.all()


def test_merge_in_place_accumulate():
    say("merge in place")
    g = torch.Generator().manual_seed(3)
    T, H = 300, 8
    po = torch.randn(T, H, 128, generator=g).to(torch.bfloat16)
    so = torch.randn(T, H, 128, generator=g).to(torch.bfloat16)
    pl = torch.randn(H, T, generator=g).float()
    sl = torch.randn(H, T, generator=g).float()
    ref_o, ref_l = O.merge_states(host(po), pl.double().numpy(), host(so), sl.double().numpy())
    p_dev, pl_dev = po.to(DEV), pl.to(DEV)
    mla.mla_merge_attn_states(p_dev, pl_dev, p_dev, pl_dev, so.to(DEV), sl.to(DEV))
    torch.cuda.synchronize()
    assert np.abs(host(p_dev) - ref_o).max() < 2e-2
    assert np.abs(pl_dev.double().cpu().numpy() - ref_l).max() < 1e-5


def test_init_partial_rows():
    say("init partial")
    T, H = 50, 3
    out = torch.full((T, H, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((H, T), 7.0, dtype=torch.float32, device=DEV)
    mla.mla_init_context_partial(out, lse, 11, 37)
    torch.cuda.synchronize()
    o, l = host(out), lse.cpu().numpy()
    assert (o[11:37] == 0).all() and np.isneginf(l[:, 11:37]).all()
    assert (o[:11] == 7).all() and (o[37:] == 7).all() and (l[:, :11] == 7).all() and (l[:, 37:] == 7).all()


# ------------------------------------------------------------------ gather


def _gather_case(wl):
    b = W.make_batch(wl, canary=True)
    plans = O.plan_mla_context_chunks(wl.context_lens, wl.workspace_rows, None, wl.split_alignment)
    kb, vb = _bits(b.k_cache), _bits(b.v_cache)
    table = b.block_table.numpy()
    d_k, d_v, d_bt = b.k_cache.to(DEV), b.v_cache.to(DEV), b.block_table.to(DEV)
    H = wl.num_heads
    for p in plans:
        n = len(p.seq_lens)
        req = torch.arange(p.request_start, p.request_end, dtype=torch.int32, device=DEV)
        st = torch.tensor(p.starts, dtype=torch.int32, device=DEV)
        off = torch.tensor(np.concatenate([[0], np.cumsum(p.seq_lens)]), dtype=torch.int32, device=DEV)
        rows = int(sum(p.seq_lens))
        cap = rows + 3
        ws_k = torch.full((cap, H, W.DK), 1.5, dtype=torch.bfloat16, device=DEV)
        ws_v = torch.full((cap, H, W.DV), 1.5, dtype=torch.bfloat16, device=DEV)
        mla.mla_gather_context(d_k, d_v, d_bt, req, st, off, rows, ws_k, ws_v)
        torch.cuda.synchronize()
        ref_k = O.gather_context_rows(kb, table, wl.block_size, list(range(p.request_start, p.request_end)),
                                      p.starts, p.seq_lens)
        ref_v = O.gather_context_rows(vb, table, wl.block_size, list(range(p.request_start, p.request_end)),
                                      p.starts, p.seq_lens)
        gk, gv = _bits(ws_k), _bits(ws_v)
        assert np.array_equal(gk[:rows], ref_k) and np.array_equal(gv[:rows], ref_v)
        # rows past num_rows are untouched
        assert (host(ws_k[rows:]) == 1.5).all() and (host(ws_v[rows:]) == 1.5).all()
        # no canary (NaN) row was gathered
        assert not np.isnan(host(ws_k[:rows])).any() and not np.isnan(host(ws_v[:rows])).any()


@pytest.mark.parametrize("idx", [1, 2])
def test_gather_named_bit_exact(idx):
    say(f"gather named {idx}")
    _gather_case(W.named_workloads()[idx])


def test_gather_random_bit_exact():
    for seed in range(12):
        wl = W.random_workload(seed, max_requests=8, max_ctx=400, max_q=4, heads=(1, 3, 8))
        say(f"gather random seed={seed} {wl}")
        _gather_case(wl)


def test_gather_bad_block_ids_give_nan_rows():
    say("gather bad block ids")
    H, B = 2, 4
    k = torch.randn(5, B, H, W.DK).to(torch.bfloat16).to(DEV)
    v = torch.randn(5, B, H, W.DV).to(torch.bfloat16).to(DEV)
    bt = torch.tensor([[1, 9, -1]], dtype=torch.int32, device=DEV)  # 9 and -1 are outside the cache
    req = torch.tensor([0], dtype=torch.int32, device=DEV)
    st = torch.tensor([0], dtype=torch.int32, device=DEV)
    off = torch.tensor([0, 14], dtype=torch.int32, device=DEV)  # rows 12,13 are past the table width
    ws_k = torch.zeros(14, H, W.DK, dtype=torch.bfloat16, device=DEV)
    ws_v = torch.zeros(14, H, W.DV, dtype=torch.bfloat16, device=DEV)
    mla.mla_gather_context(k, v, bt, req, st, off, 14, ws_k, ws_v)
    torch.cuda.synchronize()
    gk = host(ws_k)
    assert np.array_equal(gk[:4], host(k[1]))
    assert np.isnan(gk[4:]).all()


# --------------------------------------------------------------- attention


def _varlen_case(seed, q_lens, k_lens, H, causal):
    g = torch.Generator().manual_seed(seed)
    Tq, Tk = sum(q_lens), sum(k_lens)
    q = torch.randn(Tq, H, W.DK, generator=g).to(torch.bfloat16)
    k = torch.randn(Tk, H, W.DK, generator=g).to(torch.bfloat16)
    v = torch.randn(Tk, H, W.DV, generator=g).to(torch.bfloat16)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    scale = 1 / np.sqrt(W.DK)
    out = torch.full((Tq, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((H, Tq), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    dcq = torch.from_numpy(cu_q).to(DEV)
    if causal:
        mla.mla_causal_suffix_attn(dq, dk, dv, dcq, max(q_lens), scale, out, lse)
    else:
        mla.mla_context_chunk_attn(dq, dk, dv, dcq, torch.from_numpy(cu_k).to(DEV), max(q_lens), scale, out, lse)
    torch.cuda.synchronize()
    ref_o = np.zeros((Tq, H, W.DV))
    ref_l = np.full((H, Tq), -np.inf)
    qh, kh, vh = host(q), host(k), host(v)
    for i in range(len(q_lens)):
        a, b = cu_q[i], cu_q[i + 1]
        c, d = cu_k[i], cu_k[i + 1]
        o, l = O.attention_with_lse(qh[a:b], kh[c:d], vh[c:d], scale, causal=causal)
        ref_o[a:b], ref_l[:, a:b] = o, l
    vmax = max(np.abs(vh).max(), 1e-30) if vh.size else 1.0
    return check(host(out), lse.double().cpu().numpy(), ref_o, ref_l, vmax, f"seed {seed}")


@pytest.mark.parametrize("case", [
    (1, [1], [1], 1),
    (2, [5, 130, 0, 64, 257], [300, 64, 9, 0, 129], 3),   # ragged tails, empty q and empty k
    (3, [128], [4096], 2),                                  # many key tiles
    (4, [300, 17], [777, 1], 4),
    (5, [513], [65], 1),
])
def test_chunk_attention_matches_oracle(case):
    seed, ql, kl, H = case
    say(f"chunk attention {case}")
    r = _varlen_case(seed, ql, kl, H, causal=False)
    say("  ", r)


@pytest.mark.parametrize("case", [
    (11, [1], 1),
    (12, [3, 200, 1, 64, 129], 3),
    (13, [700], 2),
    (14, [128, 256, 0, 5], 2),
])
def test_suffix_attention_matches_oracle(case):
    seed, ql, H = case
    say(f"suffix attention {case}")
    r = _varlen_case(seed, ql, ql, H, causal=True)
    say("  ", r)


def _rising_case(seed, q_len, k_len, H, rate, causal):
    """Scores that grow from key tile to key tile: queries share a direction u,
    and key j carries rate * (j // 64) * u, so the running max of a query rises
    by about rate * |u|^2 * scale * log2(e) per 64-key tile (tens of log2
    units for rate 0.3), far past the point where the kernels must move their
    reference max after the first tile."""
    g = torch.Generator().manual_seed(seed)
    u = 2.0 * torch.randn(H, W.DK, generator=g)
    q = (u[None] + torch.randn(q_len, H, W.DK, generator=g)).to(torch.bfloat16)
    step = (torch.arange(k_len) // 64).float() * rate
    k = (step[:, None, None] * u[None] + torch.randn(k_len, H, W.DK, generator=g)).to(torch.bfloat16)
    v = torch.randn(k_len, H, W.DV, generator=g).to(torch.bfloat16)
    scale = 1 / np.sqrt(W.DK)
    out = torch.full((q_len, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((H, q_len), float("nan"), dtype=torch.float32, device=DEV)
    cu_q = torch.tensor([0, q_len], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, k_len], dtype=torch.int32, device=DEV)
    if causal:
        mla.mla_causal_suffix_attn(q.to(DEV), k.to(DEV), v.to(DEV), cu_q, q_len, scale, out, lse)
    else:
        mla.mla_context_chunk_attn(q.to(DEV), k.to(DEV), v.to(DEV), cu_q, cu_k, q_len, scale, out, lse)
    torch.cuda.synchronize()
    o, l = O.attention_with_lse(host(q), host(k), host(v), scale, causal=causal)
    return check(host(out), lse.double().cpu().numpy(), o, l, np.abs(host(v)).max(), f"rising seed {seed}")


@pytest.mark.parametrize("case", [
    (31, 300, 640, 2, 0.3),    # every tile raises the max by ~20 log2 units
    (32, 257, 1000, 1, 0.03),  # gentle rise: a few raises over the sequence
    (33, 64, 200, 3, -0.3),    # falling scores: the first tile holds the max
])
def test_attention_rising_scores(case):
    seed, ql, kl, H, rate = case
    say(f"chunk attention, rising scores {case}")
    say("  ", _rising_case(seed, ql, kl, H, rate, causal=False))
    say(f"suffix attention, rising scores {case}")
    say("  ", _rising_case(seed, ql, ql, H, rate, causal=True))


def test_attention_empty_keys_give_empty_state():
    say("attention with no keys")
    H = 2
    q = torch.randn(10, H, W.DK).to(torch.bfloat16).to(DEV)
    kv = torch.zeros(1, H, W.DK, dtype=torch.bfloat16, device=DEV)
    vv = torch.zeros(1, H, W.DV, dtype=torch.bfloat16, device=DEV)
    out = torch.full((10, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(H, 10, dtype=torch.float32, device=DEV)
    cu_q = torch.tensor([0, 10], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    mla.mla_context_chunk_attn(q, kv, vv, cu_q, cu_k, 10, 0.1, out, lse)
    torch.cuda.synchronize()
    assert (host(out) == 0).all() and np.isneginf(lse.cpu().numpy()).all()


def test_attention_is_deterministic():
    say("attention determinism")
    a = _varlen_case(21, [200, 33], [500, 70], 2, causal=False)
    b = _varlen_case(21, [200, 33], [500, 70], 2, causal=False)
    assert a == b


# ------------------------------------------------------- mask_empty_context


def _mask_case(query_lens, context_lens, H, D, dtype, seed, nan_rows=None):
    qsl = np.concatenate([[0], np.cumsum(query_lens)]).astype(np.int32)
    csl = np.concatenate([[0], np.cumsum(context_lens)]).astype(np.int32)
    T = int(qsl[-1])
    g = torch.Generator().manual_seed(seed)
    lse = torch.randn(H, T, generator=g)
    out = torch.randn(T, H, D, generator=g).to(dtype)
    if nan_rows is not None:
        out[nan_rows[0]:nan_rows[1]] = float("nan")
    ref_l, ref_o = lse.double().numpy().copy(), out.double().numpy().copy()
    O.mask_empty_context(ref_l, ref_o, qsl, csl)
    dl, do = lse.to(DEV), out.to(DEV)
    mla.mla_mask_empty_context(dl, do, torch.from_numpy(qsl).to(DEV), torch.from_numpy(csl).to(DEV))
    torch.cuda.synchronize()
    gl, go = dl.double().cpu().numpy(), do.double().cpu().numpy()
    assert np.array_equal(gl, ref_l) and np.array_equal(np.isnan(go), np.isnan(ref_o))
    assert np.array_equal(np.nan_to_num(go, nan=7.0), np.nan_to_num(ref_o, nan=7.0))
    return gl, go


def test_mask_empty_context_printed_test(golden):
    """The PR #49294 digest's test: rows 33..163 (request 32, no context) end
    (-inf, 0); every other value is untouched (fp32 outputs, as in the test)."""
    g = golden("empty_context_rows.json")
    say("mask_empty_context printed test")
    e0, e1 = g["empty_rows"]
    gl, go = _mask_case(g["query_lens"], g["context_lens"], g["num_heads"], g["head_dim"], torch.float32, 0,
                        nan_rows=(e0, e1))
    assert np.isneginf(gl[:, e0:e1]).all() and (go[e0:e1] == 0).all()
    assert np.isfinite(gl[:, :e0]).all() and np.isfinite(gl[:, e1:]).all()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_mask_empty_context_random(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(60, 300))  # several 64-entry search windows
    ql = [0 if rng.random() < 0.1 else int(rng.integers(1, 9)) for _ in range(n)]
    cl = [0 if rng.random() < 0.3 else int(rng.integers(1, 50)) for _ in range(n)]
    say(f"mask_empty_context random seed={seed} n={n}")
    _mask_case(ql, cl, int(rng.integers(1, 9)), 128, torch.bfloat16, seed)


@pytest.mark.parametrize("H,D,dtype", [(3, 2, torch.bfloat16), (5, 3, torch.float32), (2, 8, torch.bfloat16)])
def test_mask_empty_context_unaligned_rows(H, D, dtype):
    # rows that are not a multiple of 16 bytes take the 4-byte store path
    say(f"mask_empty_context rows of {H * D} elements ({dtype})")
    _mask_case([3, 0, 5, 2, 7], [0, 4, 0, 1, 0], H, D, dtype, 11)
