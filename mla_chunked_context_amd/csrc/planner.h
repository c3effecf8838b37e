// Internal interface of the host planner (shared by the C ABI and the
// chunked-prefill driver).  No HIP types.
#pragma once

#include <cstdint>

#include "mla_cc.h"

namespace mla {

// Receives the plan as it is produced: entries in order, and each chunk once
// it closes (its entries are the ones emitted since it opened).
struct PlanSink {
    virtual ~PlanSink() = default;
    virtual void chunk(const mla_chunk_desc& c) = 0;
    virtual void entry(int32_t start, int32_t len) = 0;
    virtual int32_t entries_so_far() const = 0;
};

// Greedy aligned packing; returns an MLA_* status.  cap <= 0 means budget.
// world/interleave > 1: context sharded over `world` ranks in runs of
// `interleave` positions; a chunk's rows are then counted in the all-gathered
// workspace, padded_rows(x) = world * interleave * ceil(x / (world * interleave)),
// and align must be a multiple of world * interleave.
int plan_chunks(const int32_t* ctx, const int32_t* qlens, int32_t n, int64_t budget, int64_t cap,
                int32_t align, PlanSink& sink, int32_t world = 1, int32_t interleave = 1);

// Rows every rank reserves for context positions [0, x) under that sharding.
inline int64_t padded_local_rows(int64_t x, int32_t world, int32_t interleave) {
    const int64_t round = static_cast<int64_t>(world) * interleave;
    return (x + round - 1) / round * interleave;
}

// prefill_tokens_with_context and the token ranges of requests without context.
int token_info(const int32_t* ctx, const int32_t* qlens, int32_t n, int64_t* prefix_num_tokens,
               int32_t* empty, int32_t cap, int32_t* num_empty);

// Window of the uniform-window scheduler: the workspace shared equally by the
// requests with context, rounded down to the alignment.  window = 0 and
// iterations = 0 when no request has context; MLA_ERR_INVALID_ARG when the
// share holds no aligned window.
int uniform_windows(const int32_t* ctx, int32_t n, int64_t budget, int32_t align, int64_t* window,
                    int32_t* iterations);

}  // namespace mla
