"""mla_chunked_prefill_no_alloc against mla_chunked_prefill, through the C ABI.

The no-allocation entry point runs the same kernels on the library's own
device buffer, with the chunk metadata carried in kernel arguments.  Two
calls in a row, the second on a smaller batch (so the buffer holds the first
call's larger state when the second starts), must each give the output and
LSE of mla_chunked_prefill on the same inputs bit for bit, and both must meet
the oracle bars.  A batch whose scratch exceeds the buffer is refused with
MLA_ERR_CAPACITY.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import check, host, oracle_inputs, record, run_prefill, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"

# the first call's batch: the tiny lengths at 128 heads (81 MiB of scratch,
# two chunks, one continuation); the second: the empty-context stress batch
# (16 heads, 4 MiB)
FIRST = W.Workload("tiny_h128", (768, 512, 512, 0), (3, 5, 7, 4), 128, 1024, 64, 64, 1.0, 601)
SECOND = W.named_workloads()[2]


def _batch(wl):
    b = W.make_batch(wl, device="cpu", canary=True)
    d = W.Batch(wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                b.block_table.to(DEV), b.num_blocks, b.spare_blocks)
    return b, d


def _no_alloc(d):
    wl = d.wl
    T, H = wl.num_tokens, wl.num_heads
    out = torch.full((T, H, W.DV), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=DEV)
    p = mla.make_prefill_params(d.q, d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, wl.context_lens,
                                wl.query_lens, wl.workspace_rows, wl.split_alignment, wl.scale, out=out, out_lse=lse)
    assert mla.mla_chunked_prefill_scratch_size(p) <= mla.NO_ALLOC_SCRATCH_BYTES
    mla.mla_chunked_prefill_no_alloc(p)
    return out, lse


def test_no_alloc_matches_chunked_prefill_two_calls():
    cases = [_batch(FIRST), _batch(SECOND)]
    say(f"no-alloc prefill: {FIRST.name} then {SECOND.name}")
    got = [_no_alloc(d) for _, d in cases]  # enqueued back to back on one stream
    torch.cuda.synchronize()
    for (b, d), (o, l) in zip(cases, got):
        wl = b.wl
        ref_o, ref_l = run_prefill(mla, d)
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"{wl.name}: output differs"
        assert torch.equal(l, ref_l), f"{wl.name}: LSE differs"
        ref = O.chunked_prefill(*oracle_inputs(b), wl.workspace_rows, wl.split_alignment, wl.scale)
        vals = np.concatenate([host(b.v_new).ravel(), np.nan_to_num(host(b.v_cache), nan=0.0).ravel()])
        res = check(host(o), l.double().cpu().numpy(), ref["out"], ref["lse"], float(np.abs(vals).max()), wl.name)
        record(f"no-alloc {wl.name} every row", res)


def test_no_alloc_refuses_batches_beyond_its_buffer():
    wl = W.named_workloads()[3]  # 5.6 GB of scratch
    T, H = wl.num_tokens, wl.num_heads
    q = torch.empty((T, H, W.DK), dtype=torch.bfloat16, device=DEV)
    p = mla.make_prefill_params(q, q, q, None, None, None, wl.context_lens, wl.query_lens, wl.workspace_rows,
                                wl.split_alignment, wl.scale)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_chunked_prefill_no_alloc(p)
    assert e.value.status == mla.MLA_ERR_CAPACITY
