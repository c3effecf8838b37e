"""Plain fp64 CPU oracle for MLA chunked-context prefill.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
package; only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may.  It shares no code with the HIP path: the two meet only
at the seeded inputs built by ``workloads``.

Sources (the vLLM pull-request digests this method is described on):
  * PR #50613 digest: per-request chunk packing (plan_mla_context_chunks,
    aligned_split_len), the ContextChunk metadata, init_mla_context_partial
    and accumulate_mla_context_chunk.
  * PR #49294 digest ("Ignore empty MLA context chunks during merge"): rows of
    requests without context must end as LSE -inf with output 0; merging two
    empty states must not give NaN.
  * PR #36540 digest ("Remove trtllm ragged mla prefills"): merge_attn_states
    with a prefix_num_tokens threshold, rows at or past it take the suffix.

Every floating-point step is float64.  Modules:
  planner    chunk packing and per-chunk metadata (integer, exact)
  attention  paged-cache gather and naive softmax attention with LSE
  merge      LSE merge, partial init/accumulate, thresholded final merge
  pipeline   the chunked prefill end to end, and the direct definition
  mask       mask_empty_context (the earlier mechanism for empty rows)
  uniform_window  the earlier equal-window scheduler, with the mask in its loop
"""
from .planner import (ChunkPlan, ContextChunk, ChunkedContextMetadata, aligned_split_len,
                      plan_mla_context_chunks, build_mla_chunked_context_metadata,
                      build_chunked_context)
from .attention import gather_context_rows, gather_row_sources, attention_with_lse
from .merge import (merge_states, merge_attn_states, init_mla_context_partial,
                    accumulate_mla_context_chunk)
from .pipeline import chunked_prefill, direct_prefill, direct_rows
from .mask import mask_empty_context
from .uniform_window import plan_uniform_windows, uniform_window_prefill, uniform_window_size

__all__ = [
    "ChunkPlan", "ContextChunk", "ChunkedContextMetadata", "aligned_split_len",
    "plan_mla_context_chunks", "build_mla_chunked_context_metadata", "build_chunked_context",
    "gather_context_rows", "gather_row_sources", "attention_with_lse", "merge_states", "merge_attn_states",
    "init_mla_context_partial", "accumulate_mla_context_chunk", "chunked_prefill",
    "direct_prefill", "direct_rows", "mask_empty_context", "plan_uniform_windows",
    "uniform_window_prefill", "uniform_window_size",
]
