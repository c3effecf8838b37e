"""Bit-exact gathers at full size, through the C ABI.

Every chunk of the homogeneous, heterogeneous and long-context workloads
(128 heads: the one-row-per-workgroup gather the benchmark times, with 64-bit
row addressing past 2^31 bytes) is gathered by mla_gather_context and
compared bit for bit, on every workspace row, with the cache rows the
oracle's index map names (oracle.gather_row_sources: physical block and slot
of each context position, PR #50613 digest, 实现拆解 item 2).  The
comparison itself runs on the device (torch index_select of the input cache
at those rows, then torch.equal on the raw bits), because the caches are tens
of GB.  Unused cache slots hold NaN canaries; rows past the chunk's row count
must stay untouched.

The DCP reorganisation is checked the same way at 128 heads: the
homogeneous workload's context sharded over 4 emulated ranks, gathered per
rank and reorganised, must equal the single-device rows bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import oracle.dcp as OD
import workloads as W
from tests.gpu_util import record, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"
GUARD = 3  # workspace rows past the chunk that must stay untouched


def _i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _bits(t, width):
    return t.reshape(-1, width).view(torch.int16)


def _check_rows(ws_k, ws_v, rows, b, src, what):
    H = b.wl.num_heads
    kflat, vflat = _bits(b.k_cache, H * W.DK), _bits(b.v_cache, H * W.DV)
    s = torch.from_numpy(src).to(DEV)
    gk, gv = _bits(ws_k, H * W.DK), _bits(ws_v, H * W.DV)
    assert torch.equal(gk[:rows], kflat.index_select(0, s)), f"{what}: K rows differ"
    assert torch.equal(gv[:rows], vflat.index_select(0, s)), f"{what}: V rows differ"
    # the oracle never maps a row onto a canary slot, so the gathered rows hold no NaN
    assert not torch.isnan(ws_k[:rows]).any().item() and not torch.isnan(ws_v[:rows]).any().item(), what
    # rows past the chunk are untouched (they hold the 1.5 fill)
    assert (ws_k[rows:rows + GUARD] == 1.5).all().item() and (ws_v[rows:rows + GUARD] == 1.5).all().item(), what


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["homogeneous", "heterogeneous", "long_context"])
def test_gather_full_size_bit_exact(name):
    wl = W.workload_by_name(name)
    say(f"gather full size {name}: H={wl.num_heads} ctx rows={sum(wl.context_lens)} W={wl.workspace_rows}")
    b = W.make_batch(wl, device=DEV, canary=True)
    H = wl.num_heads
    plans = O.plan_mla_context_chunks(list(wl.context_lens), wl.workspace_rows, None, wl.split_alignment)
    table = b.block_table.cpu().numpy()
    cap = wl.workspace_rows + GUARD
    ws_k = torch.empty((cap, H, W.DK), dtype=torch.bfloat16, device=DEV)
    ws_v = torch.empty((cap, H, W.DV), dtype=torch.bfloat16, device=DEV)
    checked = 0
    for ci, p in enumerate(plans):
        reqs = list(range(p.request_start, p.request_end))
        rows = int(sum(p.seq_lens))
        off = np.concatenate([[0], np.cumsum(p.seq_lens)])
        say(f"  chunk {ci}: requests {reqs[0]}..{reqs[-1]} rows {rows} first start {p.starts[0]}")
        ws_k.fill_(1.5)
        ws_v.fill_(1.5)
        mla.mla_gather_context(b.k_cache, b.v_cache, b.block_table, _i32(reqs), _i32(p.starts), _i32(off), rows,
                               ws_k, ws_v)
        torch.cuda.synchronize()
        src = O.gather_row_sources(table, wl.block_size, reqs, p.starts, p.seq_lens)
        assert len(src) == rows
        _check_rows(ws_k, ws_v, rows, b, src, f"{name} chunk {ci}")
        checked += rows
    assert checked == sum(wl.context_lens)
    record(f"gather {name} H={H}", {"chunks": len(plans), "rows_bit_exact": checked})


@pytest.mark.timeout(600)
def test_dcp_reorganize_full_size_bit_exact():
    wl = W.workload_by_name("homogeneous")
    world, il = 4, 1
    say(f"dcp reorganize full size {wl.name}: world={world} H={wl.num_heads}")
    b = W.make_batch(wl, device=DEV, canary=True)
    ranks = W.shard_context(b, world, il, canary=True)
    H = wl.num_heads
    chunks, st, ln, lst, lln = mla.mla_plan_dcp_context_chunks(wl.context_lens, wl.query_lens, wl.workspace_rows,
                                                               world, il, 0, wl.split_alignment)
    # the library's DCP plan is the oracle's
    oplans = OD.plan_dcp_context_chunks(list(wl.context_lens), wl.workspace_rows, wl.split_alignment, world, il)
    assert len(oplans) == len(chunks)
    table = b.block_table.cpu().numpy()
    checked = 0
    for c, op in zip(chunks, oplans):
        e0, ne = c["entry_begin"], c["num_entries"]
        reqs = list(range(c["request_begin"], c["request_end"]))
        assert reqs == list(range(op.request_start, op.request_end))
        assert list(st[e0:e0 + ne]) == list(op.starts) and list(ln[e0:e0 + ne]) == list(op.seq_lens)
        lcu = np.concatenate([[0], np.cumsum(lln[e0:e0 + ne])])
        cu = np.concatenate([[0], np.cumsum(ln[e0:e0 + ne])])
        L = int(lcu[-1])
        gk = torch.full((world * L, H, W.DK), float("nan"), dtype=torch.bfloat16, device=DEV)
        gv = torch.full((world * L, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
        for r, rc in enumerate(ranks):
            mla.mla_gather_context(rc.k_cache, rc.v_cache, rc.block_table, _i32(reqs), _i32(lst[e0:e0 + ne]),
                                   _i32(lcu), L, gk[r * L:(r + 1) * L], gv[r * L:(r + 1) * L])
        rows = int(cu[-1])
        wk = torch.full((rows + GUARD, H, W.DK), 1.5, dtype=torch.bfloat16, device=DEV)
        wv = torch.full((rows + GUARD, H, W.DV), 1.5, dtype=torch.bfloat16, device=DEV)
        mla.mla_dcp_reorganize_context(gk, gv, world, il, L, _i32(st[e0:e0 + ne]), _i32(cu), _i32(lcu), rows, wk, wv)
        torch.cuda.synchronize()
        src = O.gather_row_sources(table, wl.block_size, reqs, op.starts, op.seq_lens)
        _check_rows(wk, wv, rows, b, src, f"dcp chunk {e0}")
        checked += rows
        del gk, gv, wk, wv
    assert checked == sum(wl.context_lens)
    record(f"dcp reorganize {wl.name} H={H} world={world}", {"chunks": len(chunks), "rows_bit_exact": checked})
