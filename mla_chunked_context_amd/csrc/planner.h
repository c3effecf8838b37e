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
int plan_chunks(const int32_t* ctx, const int32_t* qlens, int32_t n, int64_t budget, int64_t cap,
                int32_t align, PlanSink& sink);

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
