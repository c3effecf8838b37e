/*
 * mla_cc.h -- C ABI of libmla_cc.so: MLA chunked-context prefill on MI355X (gfx950).
 *
 * The method (vLLM PR #50613 digest, 实现拆解 items 1-3; PR #36540 and
 * PR #49294 digests for the merge): the cached context of every prefill
 * request is packed into chunks that fit a fixed workspace of rows; each chunk
 * gathers its context K/V rows out of a paged cache, runs non-causal attention
 * of its requests' new tokens against those rows (output + log-sum-exp), and
 * LSE-merges the result into a per-token context partial.  The new tokens'
 * causal self-attention (the suffix) is then merged with the partial.
 *
 * Conventions for every call:
 *   - Return value: MLA_OK (0) or an MLA_ERR_* code; mla_status_string() gives
 *     its text.  Arguments are checked before any HIP call, so argument errors
 *     are reported without touching the GPU.  No C++ exception crosses the ABI.
 *   - "dev" pointers are device pointers owned by the caller; "host" pointers
 *     are host memory owned by the caller.  Device tensors must be 16-byte
 *     aligned and contiguous in the layout stated.  The library keeps no
 *     pointer after a call returns.
 *   - Element types: bf16 tensors are passed as void* (2 bytes per element,
 *     IEEE bfloat16 bits); LSE tensors are float (fp32) and head-major:
 *     the LSE of head h, token t is at lse[h * lse_head_stride + t].
 *   - Token-major layouts: q/k_new [T, H, 192], v_new and outputs [T, H, 128].
 *     192 = 128 no-rope + 64 rope dims (MLA_QK_HEAD_DIM), 128 = MLA_V_HEAD_DIM.
 *   - Paged cache: k_cache [num_blocks, block_size, H, 192],
 *     v_cache [num_blocks, block_size, H, 128]; context position p of request
 *     r is in block block_table[r * block_table_width + p / block_size], slot
 *     p % block_size.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls only
 *     enqueue work on it and allocate no device memory.  The only host waits
 *     are in the metadata upload of mla_chunked_prefill, mla_dcp_chunked_prefill
 *     and mla_uniform_window_prefill (see mla_chunked_prefill).
 *   - An empty attention state is LSE = -inf with output 0.  Merges select
 *     rather than multiply by zero, so the output of an empty side is never
 *     read and may hold garbage or NaN.
 */
#ifndef MLA_CC_H
#define MLA_CC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1, /* a null/misaligned pointer, a negative size, bad parameters */
    MLA_ERR_CAPACITY = 2,    /* a caller-provided buffer is too small; the needed size is reported */
    MLA_ERR_UNSUPPORTED = 3, /* a shape this build does not implement (e.g. other head dims) */
    MLA_ERR_HIP = 4          /* a HIP runtime or launch error */
};

#define MLA_QK_HEAD_DIM 192
#define MLA_V_HEAD_DIM 128
/* Most heads the attention entry points and the prefill drivers accept (the
 * kernels address one key tile of all heads with 32-bit byte offsets).  More
 * gives MLA_ERR_INVALID_ARG. */
#define MLA_MAX_HEADS 1024
#define MLA_ABI_VERSION 1
/* Size of the library's own device scratch used by mla_chunked_prefill_no_alloc (128 MiB per device). */
#define MLA_NO_ALLOC_SCRATCH_BYTES (128ull << 20)

/* Text of a status code (static storage). */
const char* mla_status_string(int status);

/* MLA_ABI_VERSION of the built library. */
int mla_abi_version(void);

/* One chunk of the plan.  Ranges are half-open.  token_begin/token_end index
 * the batch's prefill tokens (query_start_loc of request_begin / request_end).
 * Entries entry_begin .. entry_begin+num_entries-1 of the entry arrays describe
 * requests request_begin.. in order: context offset (start) and row count. */
typedef struct mla_chunk_desc {
    int32_t request_begin, request_end;
    int32_t token_begin, token_end;
    int32_t entry_begin, num_entries;
    int32_t num_rows;        /* workspace rows used: sum of the entries' row counts */
    int32_t max_seq_len;     /* longest entry */
    int32_t max_query_len;   /* longest query among the chunk's requests */
    int32_t is_continuation; /* 1 if the first entry starts past context row 0 */
} mla_chunk_desc;

/*
 * Pack every request's context rows into chunks of at most row_budget rows
 * (plan_mla_context_chunks and aligned_split_len on the PR #50613 digest,
 * 关键源码片段; invariants in 实现拆解 item 2).  Host only, pure, thread-safe,
 * allocates nothing.
 *
 * Requests are visited in order; a request's remaining rows join the open chunk
 * if they fit, otherwise the longest head of them that is a multiple of
 * split_alignment, shorter than the remainder, at most max_context_chunk and
 * fitting the free rows is placed and the chunk closes (it also closes when no
 * such head exists).  Requests with context length 0 are in no chunk and close
 * the open chunk.  Workspace rows equal context rows.
 *
 *   context_lens, query_lens  host int32[num_requests], >= 0
 *   row_budget                workspace rows per chunk
 *   max_context_chunk         cap on a split piece; <= 0 means row_budget
 *   split_alignment           split granularity (normally the cache block size)
 *   chunks / chunk_capacity   host output array; *num_chunks receives the count
 *   entry_starts, entry_seq_lens / entry_capacity
 *                             host output arrays; *num_entries receives the count
 * Pass NULL output arrays (with capacity 0) to get only the counts.  If a
 * capacity is too small the counts are still written and MLA_ERR_CAPACITY is
 * returned.  MLA_ERR_INVALID_ARG if split_alignment < 1, row_budget <
 * split_alignment, max_context_chunk < split_alignment, num_requests < 0, a
 * length is negative, or the token/row totals overflow int32.
 */
int mla_plan_context_chunks(const int32_t* context_lens, const int32_t* query_lens, int32_t num_requests,
                            int64_t row_budget, int64_t max_context_chunk, int32_t split_alignment,
                            mla_chunk_desc* chunks, int32_t chunk_capacity, int32_t* num_chunks,
                            int32_t* entry_starts, int32_t* entry_seq_lens, int32_t entry_capacity,
                            int32_t* num_entries);

/*
 * Chunk planning with the context sharded over DCP ranks (PR #50613 digest:
 * the planner's padded_rows hook in 关键源码片段; local chunks with
 * padded_local_* and local_starts in 风险与影响; DCP local chunk data in the
 * test file of 实现拆解 item 5).  The pages print neither the sharding nor
 * padded_rows; this library reads them as follows.  Position p of a request's
 * context lives on rank (p / interleave) % world_size at local index
 * (p / (interleave * world_size)) * interleave + p % interleave.  Every rank
 * reserves padded_local(x) = interleave * ceil(x / (interleave * world_size))
 * local rows for positions [0, x), and chunks are packed by rows of the
 * all-gathered workspace, padded_rows(x) = world_size * padded_local(x).
 * Otherwise as mla_plan_context_chunks; split_alignment must be a multiple of
 * world_size * interleave (else MLA_ERR_INVALID_ARG).  Per entry it also
 * returns local_start = start / world_size and the padded local length
 * padded_local(start + seq_len) - local_start (the same on every rank);
 * mla_chunk_desc.num_rows is the chunk's all-gathered rows, world_size times
 * the sum of its local lengths.  world_size = interleave = 1 gives exactly
 * mla_plan_context_chunks.
 */
int mla_plan_dcp_context_chunks(const int32_t* context_lens, const int32_t* query_lens, int32_t num_requests,
                                int64_t row_budget, int64_t max_context_chunk, int32_t split_alignment,
                                int32_t world_size, int32_t interleave, mla_chunk_desc* chunks,
                                int32_t chunk_capacity, int32_t* num_chunks, int32_t* entry_starts,
                                int32_t* entry_seq_lens, int32_t* entry_local_starts, int32_t* entry_local_lens,
                                int32_t entry_capacity, int32_t* num_entries);

/*
 * Batch-wide token fields (PR #36540 digest, 实现拆解; PR #50613 digest,
 * 实现拆解 item 1).  Host only.
 *   *prefix_num_tokens  prefill_tokens_with_context: query_start_loc just past
 *                       the last request with context (0 if none); tokens at or
 *                       past it have no context.
 *   empty_slices        host int32[2 * empty_capacity]: [begin, end) token range
 *                       of each request with no context, in order; *num_empty
 *                       receives the count (MLA_ERR_CAPACITY if it exceeds the
 *                       capacity; NULL with capacity 0 to count only).
 */
int mla_prefill_token_info(const int32_t* context_lens, const int32_t* query_lens, int32_t num_requests,
                           int64_t* prefix_num_tokens, int32_t* empty_slices, int32_t empty_capacity,
                           int32_t* num_empty);

/*
 * init_mla_context_partial (PR #50613 digest, 实现拆解 item 3): set token rows
 * [row_begin, row_end) of a context partial to the empty state: output 0 and
 * LSE -inf.
 *   out  dev bf16 [T, num_heads, head_dim] (pointer to token row 0)
 *   lse  dev fp32, head-major with lse_head_stride >= row_end
 * head_dim must be a positive multiple of 8.
 */
int mla_init_context_partial(void* out, float* lse, int64_t lse_head_stride, int64_t row_begin,
                             int64_t row_end, int32_t num_heads, int32_t head_dim, void* stream);

/*
 * Gather one chunk's context rows out of the paged cache into the workspace
 * (PR #50613 digest, 实现拆解 item 2: every context row is gathered exactly
 * once).  Workspace row w belongs to the entry i with
 * entry_row_offsets[i] <= w < entry_row_offsets[i+1]; it is context position
 * p = entry_starts[i] + (w - entry_row_offsets[i]) of request entry_request[i]:
 *   ws_k[w] = k_cache[block_table[req][p / block_size]][p % block_size]
 * and likewise ws_v, all heads at once (a bit copy).
 *   k_cache, v_cache     dev bf16 paged caches (layout above), num_blocks blocks
 *   block_table          dev int32 [num_requests, block_table_width]
 *   entry_request/starts dev int32 [num_entries]
 *   entry_row_offsets    dev int32 [num_entries + 1], nondecreasing from 0 to num_rows
 *   ws_k, ws_v           dev bf16 [>= num_rows, num_heads, 192 / 128]
 * Exactly rows 0..num_rows-1 are written.  A row whose block index falls
 * outside [0, num_blocks) or whose logical block is past block_table_width is
 * filled with NaN instead of being read.
 */
int mla_gather_context(const void* k_cache, const void* v_cache, int64_t num_blocks, int32_t block_size,
                       int32_t num_heads, const int32_t* block_table, int32_t block_table_width,
                       const int32_t* entry_request, const int32_t* entry_starts,
                       const int32_t* entry_row_offsets, int32_t num_entries, int32_t num_rows,
                       void* ws_k, void* ws_v, void* stream);

/*
 * Reorganise an all-gathered DCP workspace into request order (the step after
 * the all-gather on the PR #50613 digest's DCP path, 风险与影响; layout as in
 * mla_plan_dcp_context_chunks).  gathered_k/v stack world_size rank
 * workspaces of local_rows rows; in rank r's block, entry e's padded local
 * rows start at entry_local_offsets[e].  Output row w of entry e
 * (entry_row_offsets[e] <= w < entry_row_offsets[e+1]) is context position
 * entry_starts[e] + w - entry_row_offsets[e], copied from its rank's block.
 *   gathered_k  dev bf16 [world_size * local_rows, H, 192]   gathered_v  [.., H, 128]
 *   entry_starts, entry_row_offsets (num_entries + 1), entry_local_offsets  dev int32
 *   ws_k / ws_v dev bf16 [num_rows, H, 192] / [num_rows, H, 128]
 * A row whose source falls outside the gathered buffer is written as NaN.
 */
int mla_dcp_reorganize_context(const void* gathered_k, const void* gathered_v, int32_t num_heads,
                               int32_t world_size, int32_t interleave, int32_t local_rows,
                               const int32_t* entry_starts, const int32_t* entry_row_offsets,
                               const int32_t* entry_local_offsets, int32_t num_entries, int32_t num_rows,
                               void* ws_k, void* ws_v, void* stream);

/*
 * Varlen non-causal attention of one chunk (run_prefill_context_chunk on the
 * PR #50613 digest, 实现拆解 item 4): for sequence i, queries
 * cu_q[i]..cu_q[i+1]-1 attend to keys cu_k[i]..cu_k[i+1]-1:
 *   s_j = scale * q . k_j,  out = sum_j softmax(s)_j v_j,  lse = ln sum_j e^{s_j}.
 * bf16 MFMA products, fp32 accumulation, softmax and LSE.
 *   q    dev bf16 [Tq, H, 192]    k dev bf16 [Tk, H, 192]    v dev bf16 [Tk, H, 128]
 *   cu_q, cu_k  dev int32 [num_seqs + 1], nondecreasing from 0
 *   max_q       >= every cu_q[i+1] - cu_q[i] (rows past it are not computed)
 *   out  dev bf16 [Tq, H, 128]    lse dev fp32 [H, lse_head_stride >= Tq]
 * A sequence with no keys gets (0, -inf).  Only rows of the listed sequences
 * are written.  1 <= num_heads <= MLA_MAX_HEADS.
 */
int mla_context_chunk_attn(const void* q, const void* k, const void* v, const int32_t* cu_q,
                           const int32_t* cu_k, int32_t num_seqs, int32_t max_q, int32_t num_heads,
                           float scale, void* out, float* lse, int64_t lse_head_stride, void* stream);

/*
 * Causal self-attention of the new tokens (the suffix merged by
 * merge_attn_states on the PR #36540 digest): token i of sequence s attends to
 * tokens cu_q[s]..cu_q[s]+i (i.e. up to and including itself).
 * Layouts as mla_context_chunk_attn with k = k_new, v = v_new sharing cu_q.
 */
int mla_causal_suffix_attn(const void* q, const void* k_new, const void* v_new, const int32_t* cu_q,
                           int32_t num_seqs, int32_t max_q, int32_t num_heads, float scale, void* out,
                           float* lse, int64_t lse_head_stride, void* stream);

/*
 * merge_attn_states with prefill_tokens_with_context (PR #36540 digest,
 * 实现拆解, CUDA kernel layer; empty states per the PR #49294 digest):
 * for token t < prefix_num_tokens and each head:
 *   both LSEs -inf  -> output 0, LSE -inf (never NaN)
 *   prefix -inf     -> the suffix row (bit copy) and LSE
 *   suffix -inf     -> the prefix row (bit copy) and LSE
 *   otherwise       -> LSE-weighted average, LSE = ln(e^Lp + e^Ls)
 * for t >= prefix_num_tokens: the suffix row and LSE (prefix not read).
 *   out, prefix_out, suffix_out  dev bf16 [T, H, head_dim]; head_dim a multiple of 8
 *   out_lse (may be NULL), prefix_lse, suffix_lse  dev fp32 head-major with their strides
 * out may be the same pointer as prefix_out (and out_lse as prefix_lse): this
 * is accumulate_mla_context_chunk (PR #50613 digest, 实现拆解 item 3).  Other
 * overlaps are not allowed.
 */
int mla_merge_attn_states(void* out, float* out_lse, const void* prefix_out, const float* prefix_lse,
                          const void* suffix_out, const float* suffix_lse, int64_t num_tokens,
                          int32_t num_heads, int32_t head_dim, int64_t out_lse_stride,
                          int64_t prefix_lse_stride, int64_t suffix_lse_stride,
                          int64_t prefix_num_tokens, void* stream);

/*
 * mask_empty_context (PR #49294 digest, 实现拆解 items 1-2; test_mask_empty_context
 * in 关键源码片段), in place: for every request r whose context in this chunk
 * is empty (context_start_loc[r+1] == context_start_loc[r]), set the LSE of
 * its query rows query_start_loc[r] .. query_start_loc[r+1]-1 to -inf for all
 * heads and zero those output rows; every other row is left untouched.  Each
 * row's request is found by a wavefront-parallel search over query_start_loc
 * (no per-token metadata).  The chunked prefill above initialises the context
 * partial instead (PR #50613 digest, 实现拆解 item 3); this is the earlier
 * mechanism, kept as an operation of its own.
 *   lse                dev fp32 [H, lse_head_stride >= num_tokens]
 *   output             dev [num_tokens, H, head_dim], elements of elem_bytes (2: bf16, 4: fp32),
 *                      4-byte aligned, head_dim * elem_bytes a multiple of 4
 *   query_start_loc    dev int32 [num_requests + 1], nondecreasing from 0
 *   context_start_loc  dev int32 [num_requests + 1]
 */
int mla_mask_empty_context(float* lse, int64_t lse_head_stride, void* output, int32_t elem_bytes,
                           const int32_t* query_start_loc, const int32_t* context_start_loc,
                           int32_t num_requests, int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                           void* stream);

/* Inputs, outputs and scratch of one chunked prefill (all dev pointers are
 * caller-owned; lens are host arrays).  The scratch holds the call's chunk
 * metadata, workspace and partial results until its work on the stream has
 * completed: calls that can run at the same time (on different streams) need
 * separate scratch buffers; calls on one stream may share one. */
typedef struct mla_chunked_prefill_params {
    const void* q;              /* dev bf16 [T, H, 192] */
    const void* k_new;          /* dev bf16 [T, H, 192] */
    const void* v_new;          /* dev bf16 [T, H, 128] */
    const void* k_cache;        /* dev bf16 [num_blocks, block_size, H, 192] */
    const void* v_cache;        /* dev bf16 [num_blocks, block_size, H, 128] */
    const int32_t* block_table; /* dev int32 [num_requests, block_table_width] */
    int64_t num_blocks;
    int32_t block_size;
    int32_t block_table_width;
    const int32_t* context_lens; /* host int32 [num_requests] */
    const int32_t* query_lens;   /* host int32 [num_requests] */
    int32_t num_requests;
    int32_t num_heads;         /* 1 .. MLA_MAX_HEADS */
    float scale;
    int64_t workspace_rows;    /* row_budget of the planner */
    int64_t max_context_chunk; /* <= 0: workspace_rows */
    int32_t split_alignment;
    void* out;      /* dev bf16 [T, H, 128] */
    float* out_lse; /* dev fp32 [H, T] or NULL */
    void* scratch;  /* dev, >= mla_chunked_prefill_scratch_size bytes, 256-byte aligned */
    int64_t scratch_bytes;
} mla_chunked_prefill_params;

/* Scratch bytes mla_chunked_prefill needs for these params (host only;
 * pointer fields are not read). */
int mla_chunked_prefill_scratch_size(const mla_chunked_prefill_params* params, int64_t* bytes);

/*
 * The whole chunked-context prefill (the _compute_prefill_context loop on the
 * PR #50613 digest, 实现拆解 item 3, followed by the final merge of the
 * PR #36540 digest): plan on the host, upload the chunk metadata once, then
 * per chunk gather -> chunk attention -> accumulate into the context partial,
 * then the causal suffix attention and merge_attn_states with
 * prefix_num_tokens.  Rows of requests without context get their context
 * partial initialised to (0, -inf); a chunk's rows that no earlier chunk wrote
 * are written directly (so a single chunk covering every token needs no
 * partial initialisation or merge).  A chunk-attention launch whose longest
 * workgroup (one 256-query tile of one head against a request's rows) would
 * outlast the average load of the device's CUs (256 on MI355X) is cut along
 * the key axis:
 * each request's rows are split into 2..16 slices of at least 4096 rows (the
 * count whose longest-first schedule over the CUs, simulated on the host, is
 * shortest), one state per slice goes to the scratch, and one merge combines
 * the slices into the destination rows in fp32 (exact up to rounding: the LSE
 * combination of disjoint key sets, as merge_attn_states forms it for two).
 * The attention
 * launches are persistent: one workgroup per CU takes (sequence, head, query
 * tile) items from per-XCD queues, longest sequences first (causal: tile
 * Q-1-i paired with tile i), and moves on to the other XCDs' queues when its
 * own is empty; the queues and their counters are part of the uploaded
 * metadata.  Enqueues on `stream`; the host returns
 * once the work is enqueued.  Successive calls may overlap: the metadata is
 * staged through a ring of 4 pinned host buffers per device, each recycled
 * only after its copy has completed.  Two host waits follow from this: a call
 * that finds the next buffer's copy still pending (the fifth call in flight)
 * waits for that copy, and a buffer that must grow is freed with
 * hipHostFree (which waits for the device) and reallocated with
 * hipHostMalloc.  Neither waits for any kernel of the call itself.
 */
int mla_chunked_prefill(const mla_chunked_prefill_params* params, void* stream);

/*
 * mla_chunked_prefill for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * params, kernels and result, except:
 *   - params->scratch and params->scratch_bytes are not read.  The library's
 *     own device buffer of MLA_NO_ALLOC_SCRATCH_BYTES is used instead: one
 *     per device, created with the library's code on that device and held
 *     until the process ends; its address is looked up once per device, on
 *     the first call there.
 *   - The chunk metadata is written by small kernels that carry it in their
 *     arguments: no pinned host memory, no host copy, no host wait.
 *   - No hipMalloc, hipFree, hipHostMalloc or other allocating HIP or torch
 *     routine is called (host planning uses ordinary heap memory).
 * MLA_ERR_CAPACITY when mla_chunked_prefill_scratch_size exceeds
 * MLA_NO_ALLOC_SCRATCH_BYTES, before any work is enqueued.  Every call on a
 * device shares that device's buffer, and it keeps the last call's contents
 * (the path reads nothing it has not written in the same call): calls that
 * can run at the same time on one device (different streams, or host
 * threads enqueueing concurrently) race and must not overlap; calls on one
 * stream are ordered by it and may follow each other freely.
 */
int mla_chunked_prefill_no_alloc(const mla_chunked_prefill_params* params, void* stream);

/*
 * The uniform-window context scheduler that per-request packing replaced
 * (PR #50613 digest, 功能与动机): the workspace_rows are shared equally by
 * the requests with context, each getting a window of
 *   window = floor(floor(workspace_rows / n_ctx) / split_alignment) * split_alignment
 * rows, and iteration i covers context rows [i*window, (i+1)*window) of every
 * request; there are ceil(max context / window) iterations.  Host only, pure.
 * window = num_iterations = 0 when no request has context.
 * MLA_ERR_INVALID_ARG when the share holds no aligned window (the earlier
 * scheduler needed at least one aligned window per request with context).
 */
int mla_plan_uniform_windows(const int32_t* context_lens, int32_t num_requests, int64_t workspace_rows,
                             int32_t split_alignment, int64_t* window, int32_t* num_iterations);

/* Scratch bytes mla_uniform_window_prefill needs (host only). */
int mla_uniform_window_prefill_scratch_size(const mla_chunked_prefill_params* params, int64_t* bytes);

/*
 * The whole context prefill under the uniform-window scheduler, with the
 * PR #49294 digest's loop (实现拆解 item 2): per iteration, gather every
 * request's window, attention of the whole prefill batch against its windows,
 * mla_mask_empty_context over the iteration's result when any window is
 * empty, and (from the second iteration on) merge_attn_states of the running
 * context state with it over all tokens.  Then the causal suffix attention
 * and the final merge with prefix_num_tokens, as in mla_chunked_prefill.
 * Same params and conventions as mla_chunked_prefill (max_context_chunk is
 * not used; split_alignment rounds the window).  Its attention launches are
 * the same persistent launches as mla_chunked_prefill's (work queues per
 * iteration and for the suffix, in the uploaded metadata), without key
 * splits.  Kept to measure the scheduler change; it computes the same result
 * up to rounding.
 */
int mla_uniform_window_prefill(const mla_chunked_prefill_params* params, void* stream);

/*
 * DCP ranks emulated on one device: the context cache of each rank (its
 * positions of every request, in order, in its own paged cache and block
 * table).  Host arrays of world_size entries.
 */
typedef struct mla_dcp_ranks {
    int32_t world_size;
    int32_t interleave;
    const void* const* k_cache;        /* [r]: dev bf16 [num_blocks[r], block_size, H, 192] */
    const void* const* v_cache;        /* [r]: dev bf16 [num_blocks[r], block_size, H, 128] */
    const int32_t* const* block_table; /* [r]: dev int32 [num_requests, block_table_width[r]] */
    const int64_t* num_blocks;
    const int32_t* block_table_width;
} mla_dcp_ranks;

/* Scratch bytes mla_dcp_chunked_prefill needs (host only). */
int mla_dcp_chunked_prefill_scratch_size(const mla_chunked_prefill_params* params, const mla_dcp_ranks* ranks,
                                         int64_t* bytes);

/*
 * mla_chunked_prefill with each chunk's context rows assembled as under DCP
 * (PR #50613 digest, 风险与影响): chunks from mla_plan_dcp_context_chunks;
 * per chunk every rank gathers its padded local rows into its block of the
 * gathered workspace (which is where an all-gather would put them), then
 * mla_dcp_reorganize_context restores request order, then attention and
 * accumulate as in mla_chunked_prefill.  The params' k_cache, v_cache,
 * block_table, num_blocks and block_table_width are not used; block_size
 * applies to every rank's cache.  The result equals mla_chunked_prefill's on
 * the unsharded cache up to the rounding of a different chunking.
 */
int mla_dcp_chunked_prefill(const mla_chunked_prefill_params* params, const mla_dcp_ranks* ranks, void* stream);

/*
 * Kernel timing, a measurement aid (not part of the method).  While enabled,
 * every kernel the library launches is bracketed by a pair of HIP events
 * recorded on the launch's own stream.  mla_kernel_timing_read waits for the
 * recorded events, adds each kernel's elapsed time into times[kind] (an array
 * of MLA_KERNEL_KINDS entries, launches and total milliseconds per kind),
 * and forgets them.  Enabling costs two event records per launch; disabling
 * drops any unread events.  Thread-safe; events are per process.
 */
enum {
    MLA_KERNEL_INIT = 0,
    MLA_KERNEL_GATHER = 1,
    MLA_KERNEL_CHUNK_ATTN = 2,
    MLA_KERNEL_SUFFIX_ATTN = 3,
    MLA_KERNEL_MERGE = 4,
    MLA_KERNEL_MASK = 5,
    MLA_KERNEL_DCP_REORG = 6,
    MLA_KERNEL_KINDS = 7
};

typedef struct mla_kernel_time {
    int64_t launches;
    double total_ms;
} mla_kernel_time;

int mla_kernel_timing_enable(int enable);
int mla_kernel_timing_read(mla_kernel_time* times);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CC_H */
