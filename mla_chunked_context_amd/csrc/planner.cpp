// Host-side chunk planner and batch token fields of MLA chunked-context prefill.
//
// Packing rule (vLLM PR #50613 digest, 实现拆解 items 1-2 and the
// plan_mla_context_chunks / aligned_split_len description in 关键源码片段):
// greedy and order-preserving; a request that does not fit gets its longest
// aligned head that fits, and the chunk closes.  The chunk also closes when no
// aligned head fits, so no chunk ever exceeds the row budget, and a request
// without context closes the chunk since a chunk is a contiguous request slice.
//
// Pure host code: no HIP, no allocation beyond small stack state.
#include "planner.h"

#include <algorithm>
#include <climits>

namespace mla {

namespace {

// Longest multiple of `align` that is shorter than `rest`, at most `cap` and
// at most `room` (workspace rows equal context rows).  The digest finds it by
// binary search over multiples; with rows == positions the largest multiple is
// simply the smallest of the three limits rounded down to the grid.
int64_t aligned_head(int64_t rest, int64_t room, int64_t cap, int64_t align) {
    if (rest <= 1 || room < align) return 0;
    int64_t limit = std::min(std::min(cap, room), rest - 1);
    return (limit / align) * align;
}

}  // namespace

int plan_chunks(const int32_t* ctx, const int32_t* qlens, int32_t n, int64_t budget, int64_t cap,
                int32_t align, PlanSink& sink, int32_t world, int32_t interleave) {
    if (n < 0 || align < 1 || budget < align) return MLA_ERR_INVALID_ARG;
    if (world < 1 || interleave < 1 || align % (static_cast<int64_t>(world) * interleave) != 0)
        return MLA_ERR_INVALID_ARG;
    // workspace rows of context positions [0, x): identity on one device
    auto padded = [&](int64_t x) { return world * padded_local_rows(x, world, interleave); };
    if (cap <= 0) cap = budget;
    if (cap < align) return MLA_ERR_INVALID_ARG;
    if (n > 0 && (ctx == nullptr || qlens == nullptr)) return MLA_ERR_INVALID_ARG;
    int64_t tokens = 0;
    for (int32_t r = 0; r < n; ++r) {
        if (ctx[r] < 0 || qlens[r] < 0) return MLA_ERR_INVALID_ARG;
        tokens += qlens[r];
    }
    if (tokens > INT32_MAX || budget > INT32_MAX) return MLA_ERR_INVALID_ARG;

    // token offset of each request, computed on the fly
    int64_t tok_before = 0;  // query_start_loc of request r
    bool open = false;
    mla_chunk_desc cur{};
    int64_t rows = 0;

    auto close = [&](int64_t tok_end) {
        if (!open) return;
        cur.token_end = static_cast<int32_t>(tok_end);
        cur.num_rows = static_cast<int32_t>(rows);
        sink.chunk(cur);
        open = false;
    };

    for (int32_t r = 0; r < n; ++r) {
        const int64_t c = ctx[r];
        if (c == 0) {
            close(tok_before);
            tok_before += qlens[r];
            continue;
        }
        int64_t pos = 0;
        while (pos < c) {
            if (!open) {
                open = true;
                rows = 0;
                cur = mla_chunk_desc{};
                cur.request_begin = r;
                cur.request_end = r;
                cur.token_begin = static_cast<int32_t>(tok_before);
                cur.entry_begin = sink.entries_so_far();
                cur.is_continuation = pos > 0 ? 1 : 0;
            }
            const int64_t rest = c - pos;
            const int64_t room = budget - rows;
            int64_t take;
            bool full;
            if (padded(c) - padded(pos) <= room) {
                take = rest;
                full = false;
            } else {
                // pos and every candidate head are multiples of align, hence of
                // world * interleave, so a head's rows equal its length
                take = aligned_head(rest, room, cap, align);
                full = true;  // nothing more goes into this chunk
            }
            if (take > 0) {
                sink.entry(static_cast<int32_t>(pos), static_cast<int32_t>(take));
                cur.request_end = r + 1;
                cur.num_entries += 1;
                cur.max_seq_len = std::max<int32_t>(cur.max_seq_len, static_cast<int32_t>(take));
                cur.max_query_len = std::max<int32_t>(cur.max_query_len, qlens[r]);
                rows += padded(pos + take) - padded(pos);
                pos += take;
            }
            if (full) {
                // A chunk must hold at least one entry; the argument checks
                // (align <= budget, cap >= align) guarantee progress.
                if (cur.num_entries == 0) return MLA_ERR_INVALID_ARG;
                // token_end is query_start_loc[request_end]
                close(cur.request_end == r + 1 ? tok_before + qlens[r] : tok_before);
            }
        }
        tok_before += qlens[r];
    }
    close(tok_before);
    return MLA_OK;
}

int token_info(const int32_t* ctx, const int32_t* qlens, int32_t n, int64_t* prefix_num_tokens,
               int32_t* empty, int32_t cap, int32_t* num_empty) {
    if (n < 0 || prefix_num_tokens == nullptr || num_empty == nullptr) return MLA_ERR_INVALID_ARG;
    if (n > 0 && (ctx == nullptr || qlens == nullptr)) return MLA_ERR_INVALID_ARG;
    if (cap < 0 || (cap > 0 && empty == nullptr)) return MLA_ERR_INVALID_ARG;
    int64_t tok = 0, prefix = 0;
    int32_t count = 0;
    for (int32_t r = 0; r < n; ++r) {
        if (ctx[r] < 0 || qlens[r] < 0) return MLA_ERR_INVALID_ARG;
        const int64_t next = tok + qlens[r];
        if (next > INT32_MAX) return MLA_ERR_INVALID_ARG;
        if (ctx[r] > 0) {
            prefix = next;
        } else {
            if (count < cap) {
                empty[2 * count] = static_cast<int32_t>(tok);
                empty[2 * count + 1] = static_cast<int32_t>(next);
            }
            ++count;
        }
        tok = next;
    }
    *prefix_num_tokens = prefix;
    *num_empty = count;
    return count > cap ? MLA_ERR_CAPACITY : MLA_OK;
}

int uniform_windows(const int32_t* ctx, int32_t n, int64_t budget, int32_t align, int64_t* window,
                    int32_t* iterations) {
    if (n < 0 || budget < 1 || align < 1 || window == nullptr || iterations == nullptr) return MLA_ERR_INVALID_ARG;
    if (n > 0 && ctx == nullptr) return MLA_ERR_INVALID_ARG;
    int64_t with_ctx = 0, longest = 0;
    for (int32_t r = 0; r < n; ++r) {
        if (ctx[r] < 0) return MLA_ERR_INVALID_ARG;
        if (ctx[r] > 0) ++with_ctx;
        longest = std::max<int64_t>(longest, ctx[r]);
    }
    *window = 0;
    *iterations = 0;
    if (with_ctx == 0) return MLA_OK;
    const int64_t w = budget / with_ctx / align * align;
    if (w < 1) return MLA_ERR_INVALID_ARG;
    *window = w;
    *iterations = static_cast<int32_t>((longest + w - 1) / w);
    return MLA_OK;
}

}  // namespace mla

// ----------------------------------------------------------------------------
// C ABI (host part)

namespace {

struct ArraySink : mla::PlanSink {
    mla_chunk_desc* chunks;
    int32_t chunk_cap;
    int32_t* starts;
    int32_t* lens;
    int32_t entry_cap;
    int32_t n_chunks = 0;
    int32_t n_entries = 0;

    void chunk(const mla_chunk_desc& c) override {
        if (chunks != nullptr && n_chunks < chunk_cap) chunks[n_chunks] = c;
        ++n_chunks;
    }
    void entry(int32_t start, int32_t len) override {
        if (n_entries < entry_cap) {
            if (starts != nullptr) starts[n_entries] = start;
            if (lens != nullptr) lens[n_entries] = len;
        }
        ++n_entries;
    }
    int32_t entries_so_far() const override { return n_entries; }
};

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "ok";
        case MLA_ERR_INVALID_ARG: return "invalid argument";
        case MLA_ERR_CAPACITY: return "output capacity too small";
        case MLA_ERR_UNSUPPORTED: return "unsupported shape";
        case MLA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int mla_abi_version(void) { return MLA_ABI_VERSION; }

int mla_plan_context_chunks(const int32_t* context_lens, const int32_t* query_lens, int32_t num_requests,
                            int64_t row_budget, int64_t max_context_chunk, int32_t split_alignment,
                            mla_chunk_desc* chunks, int32_t chunk_capacity, int32_t* num_chunks,
                            int32_t* entry_starts, int32_t* entry_seq_lens, int32_t entry_capacity,
                            int32_t* num_entries) {
    if (num_chunks == nullptr || num_entries == nullptr) return MLA_ERR_INVALID_ARG;
    if (chunk_capacity < 0 || entry_capacity < 0) return MLA_ERR_INVALID_ARG;
    if ((chunk_capacity > 0 && chunks == nullptr) ||
        (entry_capacity > 0 && (entry_starts == nullptr || entry_seq_lens == nullptr)))
        return MLA_ERR_INVALID_ARG;
    ArraySink sink;
    sink.chunks = chunks;
    sink.chunk_cap = chunk_capacity;
    sink.starts = entry_starts;
    sink.lens = entry_seq_lens;
    sink.entry_cap = entry_capacity;
    const int st = mla::plan_chunks(context_lens, query_lens, num_requests, row_budget, max_context_chunk,
                                    split_alignment, sink);
    if (st != MLA_OK) return st;
    *num_chunks = sink.n_chunks;
    *num_entries = sink.n_entries;
    if (sink.n_chunks > chunk_capacity || sink.n_entries > entry_capacity) return MLA_ERR_CAPACITY;
    return MLA_OK;
}

int mla_plan_dcp_context_chunks(const int32_t* context_lens, const int32_t* query_lens, int32_t num_requests,
                                int64_t row_budget, int64_t max_context_chunk, int32_t split_alignment,
                                int32_t world_size, int32_t interleave, mla_chunk_desc* chunks,
                                int32_t chunk_capacity, int32_t* num_chunks, int32_t* entry_starts,
                                int32_t* entry_seq_lens, int32_t* entry_local_starts, int32_t* entry_local_lens,
                                int32_t entry_capacity, int32_t* num_entries) {
    if (num_chunks == nullptr || num_entries == nullptr) return MLA_ERR_INVALID_ARG;
    if (chunk_capacity < 0 || entry_capacity < 0) return MLA_ERR_INVALID_ARG;
    if ((chunk_capacity > 0 && chunks == nullptr) ||
        (entry_capacity > 0 && (entry_starts == nullptr || entry_seq_lens == nullptr ||
                                entry_local_starts == nullptr || entry_local_lens == nullptr)))
        return MLA_ERR_INVALID_ARG;
    ArraySink sink;
    sink.chunks = chunks;
    sink.chunk_cap = chunk_capacity;
    sink.starts = entry_starts;
    sink.lens = entry_seq_lens;
    sink.entry_cap = entry_capacity;
    const int st = mla::plan_chunks(context_lens, query_lens, num_requests, row_budget, max_context_chunk,
                                    split_alignment, sink, world_size, interleave);
    if (st != MLA_OK) return st;
    *num_chunks = sink.n_chunks;
    *num_entries = sink.n_entries;
    if (sink.n_chunks > chunk_capacity || sink.n_entries > entry_capacity) return MLA_ERR_CAPACITY;
    for (int32_t e = 0; e < sink.n_entries; ++e) {
        const int64_t s = entry_starts[e], len = entry_seq_lens[e];
        entry_local_starts[e] = static_cast<int32_t>(s / world_size);
        entry_local_lens[e] =
            static_cast<int32_t>(mla::padded_local_rows(s + len, world_size, interleave) - s / world_size);
    }
    return MLA_OK;
}

int mla_prefill_token_info(const int32_t* context_lens, const int32_t* query_lens, int32_t num_requests,
                           int64_t* prefix_num_tokens, int32_t* empty_slices, int32_t empty_capacity,
                           int32_t* num_empty) {
    return mla::token_info(context_lens, query_lens, num_requests, prefix_num_tokens, empty_slices,
                           empty_capacity, num_empty);
}

int mla_plan_uniform_windows(const int32_t* context_lens, int32_t num_requests, int64_t workspace_rows,
                             int32_t split_alignment, int64_t* window, int32_t* num_iterations) {
    return mla::uniform_windows(context_lens, num_requests, workspace_rows, split_alignment, window,
                                num_iterations);
}

}  // extern "C"
