"""Oracle: mask_empty_context (PR #49294 digest, 实现拆解 items 1-2 and the
test_mask_empty_context snippet in 关键源码片段).

For one chunk, request r has no context in it when its chunk context length,
context_start_loc[r+1] - context_start_loc[r], is zero.  Its query token rows
query_start_loc[r] .. query_start_loc[r+1]-1 then get LSE -inf (every head)
and output 0; every other row is left as it is.  In place.  This is the
mechanism the PR #50613 digest later removes (实现拆解 item 3); it is kept as
an alternative to initialising the context partial.
"""
from __future__ import annotations

import numpy as np


def mask_empty_context(lse, output, query_start_loc, context_start_loc):
    """lse [H, T] and output [T, H, D] (modified in place)."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    csl = np.asarray(context_start_loc, dtype=np.int64)
    for r in range(len(qsl) - 1):
        if csl[r + 1] - csl[r] == 0:
            a, b = int(qsl[r]), int(qsl[r + 1])
            lse[:, a:b] = -np.inf
            output[a:b] = 0
    return lse, output
