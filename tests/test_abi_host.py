"""C ABI checks that need no GPU: the library loads and exports every symbol
the header declares; the host planner matches the oracle bit for bit; bad
arguments are rejected before any HIP call."""
import ctypes
import math
import os
import re

import numpy as np
import torch
import pytest

import oracle as O
import workloads as W
from tests.conftest import ROOT

mla = pytest.importorskip("mla_chunked_context_amd")


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mla_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(mla.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mla.EXPORTED) == names


def test_no_alloc_prefill_refuses_batches_beyond_its_buffer_before_any_gpu_call():
    # the homogeneous batch needs 5.6 GB of scratch; the refusal comes from the
    # host checks, so no device (or device pointer) is involved
    wl = W.named_workloads()[3]
    q = torch.empty((wl.num_tokens, wl.num_heads, W.DK), dtype=torch.bfloat16, device="meta")
    p = mla.make_prefill_params(q, q, q, None, None, None, wl.context_lens, wl.query_lens, wl.workspace_rows,
                                wl.split_alignment, wl.scale)
    assert mla.mla_chunked_prefill_scratch_size(p) > mla.NO_ALLOC_SCRATCH_BYTES
    with pytest.raises(mla.MlaError) as e:
        mla.mla_chunked_prefill_no_alloc(p, stream=0)  # the default stream: never reached
    assert e.value.status == mla.MLA_ERR_CAPACITY


def test_version_and_status_strings():
    assert mla.mla_abi_version() == 1
    assert mla.mla_status_string(0) == "ok"
    assert "capacity" in mla.mla_status_string(2)


def _oracle_plan(ctx, ql, w, a, m=None):
    md = O.build_mla_chunked_context_metadata(O.plan_mla_context_chunks(ctx, w, m, a), ctx, ql)
    return md


def _assert_same_plan(ctx, ql, w, a, m=None):
    chunks, starts, lens = mla.mla_plan_context_chunks(ctx, ql, w, m or 0, a)
    md = _oracle_plan(ctx, ql, w, a, m)
    assert len(chunks) == len(md.chunks)
    for c, oc in zip(chunks, md.chunks):
        assert (c["request_begin"], c["request_end"]) == oc.request_slice
        assert (c["token_begin"], c["token_end"]) == oc.token_slice
        e0, ne = c["entry_begin"], c["num_entries"]
        assert starts[e0:e0 + ne].tolist() == oc.starts.tolist()
        assert lens[e0:e0 + ne].tolist() == oc.seq_lens.tolist()
        assert c["num_rows"] == oc.num_rows
        assert c["max_seq_len"] == oc.max_seq_len
        assert c["max_query_len"] == oc.max_query_len
        assert bool(c["is_continuation"]) == oc.is_continuation
    pnt, empty = mla.mla_prefill_token_info(ctx, ql)
    assert pnt == md.prefix_num_tokens
    assert empty == md.empty_token_slices


def test_planner_printed_example(golden):
    g = golden("tail_split_example.json")
    chunks, starts, lens = mla.mla_plan_context_chunks(g["context_lens"], g["query_lens"], g["workspace_rows"], 0, 64)
    got = [dict(starts=starts[c["entry_begin"]:c["entry_begin"] + c["num_entries"]].tolist(),
                seq_lens=lens[c["entry_begin"]:c["entry_begin"] + c["num_entries"]].tolist(),
                is_continuation=bool(c["is_continuation"])) for c in chunks]
    assert got == g["chunks"]


def test_planner_matches_oracle_named():
    for wl in W.named_workloads().values():
        _assert_same_plan(list(wl.context_lens), list(wl.query_lens), wl.workspace_rows, wl.split_alignment)


def test_planner_matches_oracle_random():
    for seed in range(10000):
        wl = W.random_workload(seed, max_requests=10, max_ctx=500, max_q=50)
        m = None
        if seed % 4 == 1 and wl.workspace_rows // 2 >= wl.split_alignment:
            m = wl.workspace_rows // 2
        _assert_same_plan(list(wl.context_lens), list(wl.query_lens), wl.workspace_rows, wl.split_alignment, m)


def test_planner_large_lens():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 64))
        ctx = [0 if rng.random() < 0.1 else int(rng.integers(1, 200_000)) for _ in range(n)]
        ql = [int(rng.integers(0, 4096)) for _ in range(n)]
        a = int(rng.choice([16, 64, 256]))
        w = int(rng.integers(a, 300_000))
        _assert_same_plan(ctx, ql, w, a)


def test_planner_rejects_bad_arguments():
    with pytest.raises(mla.MlaError) as e:
        mla.mla_plan_context_chunks([10], [1], 8, 0, 16)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG
    for args in [([10], [1], 16, 0, 0), ([10], [1], 64, 8, 16), ([-1], [1], 64, 0, 16), ([3], [-2], 64, 0, 16)]:
        with pytest.raises(mla.MlaError):
            mla.mla_plan_context_chunks(*args)


def test_planner_capacity_reporting():
    ctx = (ctypes.c_int32 * 3)(768, 512, 512)
    ql = (ctypes.c_int32 * 3)(3, 5, 7)
    nc, ne = ctypes.c_int32(0), ctypes.c_int32(0)
    one = (mla.ChunkDesc * 1)()
    st = mla._plan(ctx, ql, 3, 1024, 0, 64, one, 1, ctypes.byref(nc), None, None, 0, ctypes.byref(ne))
    # null entry arrays with capacity 0 are allowed; one chunk slot is too few
    assert st == mla.MLA_ERR_CAPACITY and nc.value == 2 and ne.value == 4
    s = (ctypes.c_int32 * 8)()
    n = (ctypes.c_int32 * 8)()
    st = mla._plan(ctx, ql, 3, 1024, 0, 64, one, 1, ctypes.byref(nc), s, n, 8, ctypes.byref(ne))
    assert st == mla.MLA_ERR_CAPACITY and nc.value == 2 and ne.value == 4


def test_device_calls_reject_bad_arguments_without_gpu():
    """Argument checks run before any HIP call, so they work on a CPU-only host."""
    f = mla._lib
    # null pointers with work to do
    assert f.mla_merge_attn_states(None, None, None, None, None, None, ctypes.c_int64(4), 2, 128, ctypes.c_int64(4),
                                   ctypes.c_int64(4), ctypes.c_int64(4), ctypes.c_int64(4), None) == 1
    # head_dim not a multiple of 8
    assert f.mla_init_context_partial(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_int64(8),
                                      ctypes.c_int64(0), ctypes.c_int64(4), 2, 12, None) == 1
    # misaligned output pointer
    assert f.mla_init_context_partial(ctypes.c_void_p(258), ctypes.c_void_p(256), ctypes.c_int64(8),
                                      ctypes.c_int64(0), ctypes.c_int64(4), 2, 16, None) == 1
    # non-positive scale
    assert f.mla_context_chunk_attn(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                                    ctypes.c_void_p(256), ctypes.c_void_p(256), 1, 4, 2, ctypes.c_float(0.0),
                                    ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_int64(4), None) == 1
    # gather with rows but no entries
    assert f.mla_gather_context(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_int64(4), 16, 2,
                                ctypes.c_void_p(256), 4, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                ctypes.c_void_p(256), 0, 8, ctypes.c_void_p(256), ctypes.c_void_p(256), None) == 1
    # empty work is a no-op success, no HIP call
    assert f.mla_merge_attn_states(None, None, None, None, None, None, ctypes.c_int64(0), 2, 128, ctypes.c_int64(0),
                                   ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0), None) == 0


def test_head_count_bound():
    # the attention kernels address a key tile of all heads with 32-bit byte
    # offsets; head counts past MLA_MAX_HEADS are refused before any HIP call
    f = mla._lib
    args = lambda h: (ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),  # noqa: E731
                      ctypes.c_void_p(256), 1, 4, h, ctypes.c_float(0.07), ctypes.c_void_p(256),
                      ctypes.c_void_p(256), ctypes.c_int64(4), None)
    assert f.mla_context_chunk_attn(*args(1025)) == mla.MLA_ERR_INVALID_ARG
    wl = W.named_workloads()[1]
    q = torch.empty((wl.num_tokens, 1025, W.DK), dtype=torch.bfloat16, device="meta")
    p = mla.make_prefill_params(q, q, q, None, None, None, wl.context_lens, wl.query_lens, wl.workspace_rows,
                                wl.split_alignment, wl.scale)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_chunked_prefill_scratch_size(p)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG


def test_prefill_scratch_size_and_param_checks():
    wl = W.named_workloads()[5]
    p = mla.ChunkedPrefillParams()
    ctx = np.asarray(wl.context_lens, dtype=np.int32)
    ql = np.asarray(wl.query_lens, dtype=np.int32)
    p.context_lens, p.query_lens, p.num_requests = ctx.ctypes.data, ql.ctypes.data, 4
    p.num_heads, p.block_size, p.block_table_width, p.num_blocks = 128, 64, 2048, 8192
    p.scale, p.workspace_rows, p.split_alignment = wl.scale, wl.workspace_rows, 64
    n = mla.mla_chunked_prefill_scratch_size(p)
    T, H, Wr = 32768, 128, 65536
    expect_min = Wr * H * 640 + 2 * T * H * (256 + 4) + 8192 * H * 260
    assert expect_min <= n <= expect_min + 64 * 4096
    p.scratch_bytes = n - 1
    # too-small scratch is caught before any HIP call... after pointer checks
    with pytest.raises(mla.MlaError):
        mla.mla_chunked_prefill(p, stream=0)
    p.split_alignment = 0
    with pytest.raises(mla.MlaError):
        mla.mla_chunked_prefill_scratch_size(p)


def _schedule_length(q_lens, k_rows, heads, cus, slices, slice_tiles):
    """Tile steps of list scheduling the launch's workgroups on `cus` CUs,
    longest first, each costing its key tiles (of its slice) plus one: the
    workgroups of one cost go one per CU in whole rounds, the rest to the
    least loaded CUs."""
    count = {}
    for q, k in zip(q_lens, k_rows):
        if q <= 0:
            continue
        kt = (k + 63) // 64
        for s in range(slices):
            c = kt if slices == 1 else max(0, min(kt - s * slice_tiles, slice_tiles))
            count[c + 1] = count.get(c + 1, 0) + (q + 255) // 256 * heads
    loads = [0] * cus
    for c in sorted(count, reverse=True):
        rounds, rest = divmod(count[c], cus)
        loads = sorted(x + rounds * c for x in loads)
        loads = [x + c for x in loads[:rest]] + loads[rest:]
    return max(loads)


def _split_rule(q_lens, k_rows, heads, cus=256):
    """Key slices of one chunk-attention launch, restated: no split while the
    longest workgroup (one 256-query tile against a sequence's key tiles)
    stays within 1.2x the average CU load; otherwise the S in 2..16 (slices
    of at least 64 whole tiles) whose list schedule is shortest, taken only
    when 3% shorter than the best smaller S."""
    tiles = [(k + 63) // 64 for q, k in zip(q_lens, k_rows) if q > 0]
    work = sum((q + 255) // 256 * ((k + 63) // 64) * heads for q, k in zip(q_lens, k_rows) if q > 0)
    if not tiles or work == 0:
        return 1
    longest, avg = max(tiles), work / cus
    if longest <= 1.2 * avg:
        return 1
    best, best_len = 1, _schedule_length(q_lens, k_rows, heads, cus, 1, 0)
    for s in range(2, 17):
        if longest // s < 64:
            break
        per = -(-longest // s)
        if -(-longest // per) != s:
            continue
        n = _schedule_length(q_lens, k_rows, heads, cus, s, per)
        if n < 0.97 * best_len:
            best, best_len = s, n
    return best


def _scratch(ctx, q, heads, workspace_rows=32768):
    p = mla.ChunkedPrefillParams()
    c = np.asarray(ctx, dtype=np.int32)
    ql = np.asarray(q, dtype=np.int32)
    p.context_lens, p.query_lens, p.num_requests = c.ctypes.data, ql.ctypes.data, len(ctx)
    p.num_heads, p.block_size, p.block_table_width, p.num_blocks = heads, 64, 1024, 1024
    p.scale, p.workspace_rows, p.split_alignment = 0.07, workspace_rows, 64
    return mla.mla_chunked_prefill_scratch_size(p)


@pytest.mark.parametrize("q,heads,ctx_split", [(20, 4, 30000), (300, 16, 20000), (600, 128, 20000), (5, 2, 8192)])
def test_key_split_scratch_follows_the_split_rule(q, heads, ctx_split):
    # one request in one chunk either way: only the context length differs, so
    # the scratch differs by exactly the key-slice states of the split launch,
    # S x q rows x heads x (256 B output + 4 B LSE), each part 256-byte aligned
    s = _split_rule([q], [ctx_split], heads)
    assert _split_rule([q], [3000], heads) == 1
    diff = _scratch([ctx_split], [q], heads) - _scratch([3000], [q], heads)
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    expect = 0 if s == 1 else up(s * q * heads * 256) + up(s * heads * q * 4)
    assert diff == expect, (s, diff, expect)


def test_key_split_balances_a_mixed_launch():
    # one GPU's 16-head share of a chunk of the heterogeneous batch: two long
    # requests and a short one.  Cutting at the average load (2 slices) leaves
    # 384 equal workgroups for 256 CUs, two rounds on half of them; the list
    # schedule picks 4 slices, which spread over the CUs in three even rounds
    q, ctx, heads = [1905, 56, 1008], [67004, 414, 63616], 16
    s = _split_rule(q, ctx, heads)
    assert s == 4
    assert _schedule_length(q, ctx, heads, 256, 4, 262) < 0.8 * _schedule_length(q, ctx, heads, 256, 2, 524)
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    rows = sum(q)
    diff = _scratch(ctx, q, heads, 200000) - _scratch([3000, 414, 3000], q, heads, 200000)
    assert diff == up(s * rows * heads * 256) + up(s * heads * rows * 4)


def test_kernel_kinds_match_header():
    text = open(os.path.join(ROOT, "include", "mla_cc.h")).read()
    kinds = re.findall(r"MLA_KERNEL_([A-Z_]+) = (\d+)", text)
    names = {int(v): k.lower() for k, v in kinds if k != "KINDS"}
    assert len(mla.KERNEL_KINDS) == int(dict(kinds)["KINDS"])
    assert [names[i] for i in range(len(names))] == list(mla.KERNEL_KINDS)


def test_timing_read_without_launches():
    mla.mla_kernel_timing_enable(True)
    t = mla.mla_kernel_timing_read()
    mla.mla_kernel_timing_enable(False)
    assert all(v == (0, 0.0) for v in t.values())


def test_mask_rejects_bad_arguments_without_gpu():
    f = mla._lib
    assert f.mla_mask_empty_context(ctypes.c_void_p(256), ctypes.c_int64(8), ctypes.c_void_p(256), 3,
                                    ctypes.c_void_p(256), ctypes.c_void_p(256), 2, ctypes.c_int64(8), 2, 16,
                                    None) == 1  # element size 3
    assert f.mla_mask_empty_context(None, ctypes.c_int64(8), ctypes.c_void_p(256), 4, ctypes.c_void_p(256),
                                    ctypes.c_void_p(256), 2, ctypes.c_int64(8), 2, 16, None) == 1


def test_uniform_windows_match_oracle():
    rng = np.random.default_rng(11)
    for _ in range(3000):
        n = int(rng.integers(0, 40))
        ctx = [0 if rng.random() < 0.3 else int(rng.integers(1, 5000)) for _ in range(n)]
        a = int(rng.choice([1, 16, 64]))
        n_ctx = sum(c > 0 for c in ctx)
        rows = int(rng.integers(1, max(2, n_ctx) * a * 50))
        try:
            w_ref, _, lens = O.plan_uniform_windows(ctx, rows, a)
        except ValueError:
            with pytest.raises(mla.MlaError):
                mla.mla_plan_uniform_windows(ctx, rows, a)
            continue
        assert mla.mla_plan_uniform_windows(ctx, rows, a) == (w_ref, len(lens)), (ctx, rows, a)
    for wl in W.named_workloads().values():
        if wl.name == "empty_context_stress":
            continue  # 33 requests with context share 256 rows: no 16-row window
        w_ref, _, lens = O.plan_uniform_windows(wl.context_lens, wl.workspace_rows, wl.split_alignment)
        assert mla.mla_plan_uniform_windows(wl.context_lens, wl.workspace_rows, wl.split_alignment) == \
            (w_ref, len(lens))


def test_uniform_window_prefill_host_checks():
    wl = W.named_workloads()[4]
    p = mla.ChunkedPrefillParams()
    ctx = np.asarray(wl.context_lens, dtype=np.int32)
    ql = np.asarray(wl.query_lens, dtype=np.int32)
    p.context_lens, p.query_lens, p.num_requests = ctx.ctypes.data, ql.ctypes.data, len(ctx)
    p.num_heads, p.block_size, p.block_table_width, p.num_blocks = 128, 64, 4096, 8192
    p.scale, p.workspace_rows, p.split_alignment = wl.scale, wl.workspace_rows, 64
    n = mla.mla_uniform_window_prefill_scratch_size(p)
    T, H = wl.num_tokens, 128
    w, _ = mla.mla_plan_uniform_windows(wl.context_lens, wl.workspace_rows, 64)
    n_ctx = sum(c > 0 for c in wl.context_lens)
    assert n >= 4 * T * H * 260 and n <= 4 * T * H * 260 + n_ctx * w * H * 640 + 64 * 4096
    p.scratch_bytes = n
    with pytest.raises(mla.MlaError):  # null device pointers
        mla.mla_uniform_window_prefill(p, stream=0)
    p.workspace_rows = n_ctx * 64 - 1  # below one aligned window per request
    with pytest.raises(mla.MlaError):
        mla.mla_uniform_window_prefill_scratch_size(p)


def test_dcp_planner_matches_oracle():
    import oracle.dcp as OD
    rng = np.random.default_rng(12)
    cases = [(1, 1), (2, 1), (4, 1), (8, 1), (2, 4), (4, 2), (3, 1)]
    for _ in range(1500):
        world, il = cases[int(rng.integers(0, len(cases)))]
        a = world * il * int(rng.choice([1, 2, 8]))
        n = int(rng.integers(1, 12))
        ctx = [0 if rng.random() < 0.2 else int(rng.integers(1, 5000)) for _ in range(n)]
        ql = [int(rng.integers(0, 50)) for _ in range(n)]
        w = int(rng.integers(a, 6000))
        chunks, st, ln, lst, lln = mla.mla_plan_dcp_context_chunks(ctx, ql, w, world, il, 0, a)
        plans = OD.plan_dcp_context_chunks(ctx, w, a, world, il)
        assert len(chunks) == len(plans)
        for c, pl in zip(chunks, plans):
            e0, e1 = c["entry_begin"], c["entry_begin"] + c["num_entries"]
            ls, lens, cu = OD.dcp_local_entries(pl, world, il)
            assert (c["request_begin"], c["request_end"]) == (pl.request_start, pl.request_end)
            assert list(st[e0:e1]) == pl.starts and list(ln[e0:e1]) == pl.seq_lens
            assert list(lst[e0:e1]) == ls and list(lln[e0:e1]) == lens
            assert c["num_rows"] == world * int(cu[-1])
    with pytest.raises(mla.MlaError):
        mla.mla_plan_dcp_context_chunks([100], [1], 256, 4, 8, 0, 16)  # 16 is not a multiple of 32


def test_dcp_entry_points_reject_bad_arguments_without_gpu():
    f = mla._lib
    assert f.mla_dcp_reorganize_context(None, None, 0, 2, 1, 4, None, None, None, 1, 4, None, None, None) == 1
    assert f.mla_dcp_reorganize_context(None, None, 2, 2, 1, 4, None, None, None, 1, 0, None, None, None) == 0
    wl = W.named_workloads()[1]
    p = mla.ChunkedPrefillParams()
    ctx = np.asarray(wl.context_lens, dtype=np.int32)
    ql = np.asarray(wl.query_lens, dtype=np.int32)
    p.context_lens, p.query_lens, p.num_requests = ctx.ctypes.data, ql.ctypes.data, len(ctx)
    p.num_heads, p.block_size = wl.num_heads, wl.block_size
    p.scale, p.workspace_rows, p.split_alignment = wl.scale, wl.workspace_rows, 64
    ranks = mla.DcpRanks()
    ranks.world_size, ranks.interleave = 4, 1
    n = mla.mla_dcp_chunked_prefill_scratch_size(p, ranks)
    assert n >= mla.mla_chunked_prefill_scratch_size(p)
    p.scratch_bytes = n
    with pytest.raises(mla.MlaError):  # null device pointers
        mla.mla_dcp_chunked_prefill(p, ranks, stream=0)
    ranks.world_size = 3  # 64 is not a multiple of 3
    with pytest.raises(mla.MlaError):
        mla.mla_dcp_chunked_prefill_scratch_size(p, ranks)
