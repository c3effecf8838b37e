"""Edge cases of the whole path through the C ABI, on each driver: the
per-request packer (mla_chunked_prefill), the equal-window scheduler
(mla_uniform_window_prefill) and the context assembled from two emulated DCP
ranks (mla_dcp_chunked_prefill). Every output row and LSE is compared with the
oracle's chunked path, which the CPU tests pin to the direct definition. Cache
slots outside the contexts and all scratch start as NaN.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import check, host, oracle_inputs, run_dcp_prefill, run_prefill, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_chunked_context_amd as mla  # noqa: E402

DEV = "cuda:0"

# (name, context_lens, query_lens, H, workspace_rows, alignment, block_size, scale, seed)
EDGE = [
    # no request has context: no chunk, every row is the causal suffix alone
    W.Workload("no_context", (0, 0, 0), (5, 1, 7), 2, 256, 16, 16, 1.0, 501),
    # contexts but no new tokens: nothing to write, nothing launched
    W.Workload("no_tokens", (100, 40), (0, 0), 2, 256, 16, 16, 1.0, 502),
    # no requests at all
    W.Workload("empty_batch", (), (), 2, 256, 16, 16, 1.0, 507),
    # each context fills the workspace exactly: two chunks, no split
    W.Workload("exact_fit", (256, 256), (3, 2), 2, 256, 16, 16, 1.0, 503),
    # one row over: a 256-row head, then a continuation of a single row
    W.Workload("one_over", (257, 33), (4, 4), 2, 256, 16, 16, 1.0, 504),
    # contexts shorter than the alignment (one chunk, tail-only tiles)
    W.Workload("below_align", (5, 3, 1), (2, 2, 2), 2, 64, 64, 16, 1.0, 505),
    # one new token against a context split into six chunks
    W.Workload("one_query_long", (3000,), (1,), 3, 512, 64, 64, 1.0, 506),
    # requests with context but no new tokens between ones that have both
    W.Workload("zero_query_with_context", (300, 200, 0, 50), (0, 4, 3, 0), 2, 256, 16, 16, 1.0, 508),
    # the most heads the library accepts (MLA_MAX_HEADS): row strides of 384 KB (K) and 256 KB (V)
    W.Workload("max_heads", (100, 0, 37), (40, 3, 33), 1024, 128, 16, 16, 1.0, 509),
    # 500 requests in one chunk: the persistent attention launches' work tables do not fit
    # their LDS copy, so chunk and suffix attention take the one-workgroup-per-tile form
    W.Workload("many_requests", tuple(int(x) for x in np.random.default_rng(510).integers(1, 41, 500)),
               tuple(int(x) for x in np.random.default_rng(511).integers(1, 4, 500)), 2, 16384, 4, 4, 1.0, 510),
]


def _reference(b):
    wl = b.wl
    return O.chunked_prefill(*oracle_inputs(b), wl.workspace_rows, wl.split_alignment, wl.scale)


def _to_device(b):
    return W.Batch(b.wl, b.q.to(DEV), b.k_new.to(DEV), b.v_new.to(DEV), b.k_cache.to(DEV), b.v_cache.to(DEV),
                   b.block_table.to(DEV), b.num_blocks, b.spare_blocks)


def _vmax(b):
    vals = np.concatenate([host(b.v_new).ravel(), np.nan_to_num(host(b.v_cache), nan=0.0).ravel()])
    return float(np.abs(vals).max(initial=0.0)) or 1.0


def _uniform_window_possible(wl):
    n_ctx = sum(c > 0 for c in wl.context_lens)
    return n_ctx == 0 or wl.workspace_rows // n_ctx // wl.split_alignment > 0


@pytest.mark.parametrize("path", ["chunked", "uniform_window", "dcp"])
@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_edge_case(wl, path):
    say(f"edge case {wl.name} on {path}: ctx={wl.context_lens} q={wl.query_lens} W={wl.workspace_rows}")
    b = W.make_batch(wl, device="cpu", canary=True)
    ref = _reference(b)
    d = _to_device(b)
    if path == "dcp":
        ranks = W.shard_context(d, 2, 1)
        out, lse = run_dcp_prefill(mla, d, ranks, 1)
    else:
        if path == "uniform_window" and not _uniform_window_possible(wl):
            # the equal share rounds down to no aligned window: rejected before any launch
            with pytest.raises(mla.MlaError):
                run_prefill(mla, d, path=path)
            return
        out, lse = run_prefill(mla, d, path=path)
    assert out.shape == (wl.num_tokens, wl.num_heads, W.DV)
    say("  ", check(host(out), lse.double().cpu().numpy(), ref["out"], ref["lse"], _vmax(b), f"{wl.name}/{path}"))
